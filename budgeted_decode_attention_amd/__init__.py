"""Heavy-hitter KV-cache eviction fused into decode attention, native to MI355X.

The compute path is libkvevict.so (HIP kernels for gfx950 behind a C ABI,
include/kvevict.h); ``binding`` is its thin ctypes binding and ``build``
compiles it in-tree.
"""

from .binding import (KVCache, KVEvictError, kvevict_capacity, kvevict_create,  # noqa: F401
                      kvevict_decode_step, kvevict_destroy, kvevict_kept_indices, kvevict_position,
                      kvevict_prefill, kvevict_workspace_size, load_library)
