"""ctypes binding of libkvevict (include/kvevict.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libkvevict.so.  torch provides device memory (the workspace and the caller's
tensors) and the current HIP stream.  If the shared library is missing this
module raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvevict.so")

KVE_OK, KVE_EINVAL, KVE_ESTATE, KVE_ENOMEM, KVE_EDEVICE, KVE_EUNSUPPORTED = range(6)
KVE_F32, KVE_F16, KVE_BF16 = 0, 1, 2
KVE_FULL, KVE_H2O, KVE_LOCAL, KVE_SPECIAL, KVE_HASH, KVE_PERSIST, KVE_ADAPTIVE = 0, 1, 2, 3, 4, 5, 6

DTYPE_CODES = {torch.float32: KVE_F32, torch.float16: KVE_F16, torch.bfloat16: KVE_BF16}
CODE_DTYPES = {v: k for k, v in DTYPE_CODES.items()}

EXPORTED = ("kvevict_workspace_size", "kvevict_create", "kvevict_destroy", "kvevict_prefill",
            "kvevict_decode_step", "kvevict_decode_step_noalloc", "kvevict_kept_indices", "kvevict_unit_policies", "kvevict_cache_rows",
            "kvevict_capacity", "kvevict_position", "kvevict_stream_read", "kvevict_status_string",
            "kvevict_last_error")


class KVEvictError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(what)


class kve_config(ctypes.Structure):
    _fields_ = [
        ("layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("max_context", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("policy", ctypes.POINTER(ctypes.c_int32)), ("heavy", ctypes.POINTER(ctypes.c_int32)),
        ("recent", ctypes.POINTER(ctypes.c_int32)),
        ("vocab", ctypes.c_int32), ("keep_token_bitmap", ctypes.POINTER(ctypes.c_uint32)),
        ("sketch_bits", ctypes.c_int32), ("lsh_proj_bf16", ctypes.POINTER(ctypes.c_uint16)),
        ("history", ctypes.POINTER(ctypes.c_int32)),
        ("special_token_bitmap", ctypes.POINTER(ctypes.c_uint32)),
        ("punct_token_bitmap", ctypes.POINTER(ctypes.c_uint32)),
        ("profile_rows", ctypes.c_int32), ("profile_threshold", ctypes.c_float),
        ("cache_bits", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libkvevict.so (built in-tree by budgeted_decode_attention_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m budgeted_decode_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(kve_config)
    sig = {
        "kvevict_workspace_size": (i32, [cfgp, ctypes.POINTER(sz)]),
        "kvevict_create": (i32, [cfgp, vp, sz, ctypes.POINTER(vp)]),
        "kvevict_destroy": (i32, [vp]),
        "kvevict_prefill": (i32, [vp, i32, i32, vp, vp, vp, vp, vp, vp]),
        "kvevict_decode_step": (i32, [vp, i32, vp, vp, vp, vp, vp, vp, vp]),
        "kvevict_decode_step_noalloc": (i32, [vp, i32, vp, vp, vp, vp, vp, vp, vp]),
        "kvevict_kept_indices": (i32, [vp, i32, vp, vp, vp, vp]),
        "kvevict_unit_policies": (i32, [vp, i32, vp, vp]),
        "kvevict_cache_rows": (i32, [vp, i32, vp, vp, vp, vp, vp]),
        "kvevict_capacity": (i32, [vp, i32]),
        "kvevict_position": (i32, [vp, i32]),
        "kvevict_stream_read": (i32, [vp, sz, vp, vp]),
        "kvevict_status_string": (ctypes.c_char_p, [i32]),
        "kvevict_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != KVE_OK:
        lib = load_library()
        msg = lib.kvevict_last_error().decode()
        name = lib.kvevict_status_string(status).decode()
        raise KVEvictError(status, f"{what}: {name}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def keep_bitmap(keep_ids: Sequence[int], vocab: int) -> np.ndarray:
    bm = np.zeros((vocab + 31) // 32, dtype=np.uint32)
    for i in keep_ids:
        if 0 <= i < vocab:
            bm[i >> 5] |= np.uint32(1 << (i & 31))
    return bm


def make_config(layers: int, batch: int, heads: int, head_dim: int, max_context: int, dtype: torch.dtype,
                policy, heavy, recent, softmax_scale: float = 0.0, keep_ids: Sequence[int] = (),
                vocab: int = 0, proj: Optional[torch.Tensor] = None, history=None,
                special_ids: Optional[Sequence[int]] = None, punct_ids: Optional[Sequence[int]] = None,
                profile_rows: int = 0, profile_threshold: float = 0.0, cache_bits: int = 0):
    """Returns (kve_config, keepalive) -- keepalive holds the host tables.

    history: per-head history windows [layers * heads] (PERSIST heads), or None.
    special_ids, punct_ids, profile_rows, profile_threshold: ADAPTIVE heads.
    cache_bits: 0 (rows in the storage dtype) or 4 (4-bit slots).
    """
    pol = np.ascontiguousarray(np.asarray(policy, dtype=np.int32).reshape(-1))
    hv = np.ascontiguousarray(np.asarray(heavy, dtype=np.int32).reshape(-1))
    rc = np.ascontiguousarray(np.asarray(recent, dtype=np.int32).reshape(-1))
    keep = [pol, hv, rc]
    cfg = kve_config()
    cfg.layers, cfg.batch, cfg.heads, cfg.head_dim = layers, batch, heads, head_dim
    cfg.max_context, cfg.dtype, cfg.softmax_scale = max_context, DTYPE_CODES[dtype], softmax_scale
    cfg.policy = pol.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    cfg.heavy = hv.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    cfg.recent = rc.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    cfg.cache_bits = cache_bits
    if vocab:
        bm = keep_bitmap(keep_ids, vocab)
        keep.append(bm)
        cfg.vocab = vocab
        cfg.keep_token_bitmap = bm.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))
    if proj is not None:
        p = proj.detach().to("cpu").contiguous()
        if p.dtype != torch.bfloat16:
            raise ValueError("projection must be bfloat16")
        if p.dim() == 2:
            p = p.unsqueeze(0).expand(layers, -1, -1).contiguous()
        bits = np.ascontiguousarray(p.view(torch.int16).numpy().view(np.uint16).reshape(-1))
        keep.append(bits)
        cfg.sketch_bits = int(p.shape[-1])
        cfg.lsh_proj_bf16 = bits.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))
    if history is not None:
        hw = np.ascontiguousarray(np.asarray(history, dtype=np.int32).reshape(-1))
        keep.append(hw)
        cfg.history = hw.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    if special_ids is not None or punct_ids is not None:
        if not vocab:
            raise ValueError("special_ids / punct_ids need vocab")
        cfg.vocab = vocab
        for field, ids_ in (("special_token_bitmap", special_ids or ()), ("punct_token_bitmap", punct_ids or ())):
            bm = keep_bitmap(ids_, vocab)
            keep.append(bm)
            setattr(cfg, field, bm.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)))
        cfg.profile_rows, cfg.profile_threshold = profile_rows, profile_threshold
    return cfg, keep


# ---- thin wrappers with the C names ----------------------------------------------------------

def kvevict_workspace_size(cfg: kve_config) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().kvevict_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "kvevict_workspace_size")
    return n.value


def kvevict_create(cfg: kve_config, workspace: torch.Tensor) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().kvevict_create(ctypes.byref(cfg), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         ctypes.byref(h)), "kvevict_create")
    return h


def kvevict_destroy(h) -> None:
    _check(load_library().kvevict_destroy(h), "kvevict_destroy")


def kvevict_prefill(h, layer: int, prompt_len: int, q, k, v, token_ids=None, out=None, stream=None) -> None:
    _check(load_library().kvevict_prefill(h, layer, prompt_len, _ptr(q), _ptr(k), _ptr(v), _ptr(token_ids),
                                          _ptr(out), _stream(stream)), "kvevict_prefill")


def kvevict_decode_step(h, layer: int, q, k, v, token_ids=None, out=None, evicted_pos=None, stream=None) -> None:
    _check(load_library().kvevict_decode_step(h, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(token_ids), _ptr(out),
                                              _ptr(evicted_pos), _stream(stream)), "kvevict_decode_step")


def kvevict_decode_step_noalloc(h, layer: int, q, k, v, token_ids=None, out=None, evicted_pos=None,
                                stream=None) -> None:
    _check(load_library().kvevict_decode_step_noalloc(h, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(token_ids),
                                                      _ptr(out), _ptr(evicted_pos), _stream(stream)),
           "kvevict_decode_step_noalloc")


def kvevict_kept_indices(h, layer: int, pos_out, count_out, scores_out=None, stream=None) -> None:
    _check(load_library().kvevict_kept_indices(h, layer, _ptr(pos_out), _ptr(count_out), _ptr(scores_out),
                                               _stream(stream)), "kvevict_kept_indices")


def kvevict_unit_policies(h, layer: int, choice_out, stream=None) -> None:
    _check(load_library().kvevict_unit_policies(h, layer, _ptr(choice_out), _stream(stream)),
           "kvevict_unit_policies")


def kvevict_cache_rows(h, layer: int, k_out, v_out, k_scale_out=None, v_scale_out=None, stream=None) -> None:
    _check(load_library().kvevict_cache_rows(h, layer, _ptr(k_out), _ptr(v_out), _ptr(k_scale_out),
                                             _ptr(v_scale_out), _stream(stream)), "kvevict_cache_rows")


def kvevict_capacity(h, layer: int) -> int:
    return int(load_library().kvevict_capacity(h, layer))


def kvevict_position(h, layer: int) -> int:
    return int(load_library().kvevict_position(h, layer))


def kvevict_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Streaming read of the whole of `src` (measurement aid; see the header)."""
    if not src.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < 1 or src.device != sink.device:
        raise ValueError("src must be contiguous and sink an int32 tensor of >= 1 element on the same device")
    _check(load_library().kvevict_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                              _stream(stream)), "kvevict_stream_read")


# ---- convenience object ------------------------------------------------------------------------

class KVCache:
    """One handle plus its workspace: the caches of every layer of a model.

    Tensor arguments are validated for shape, dtype, device and contiguity
    here (the C ABI sees raw pointers only), then passed through.
    """

    def __init__(self, layers: int, batch: int, heads: int, head_dim: int, max_context: int,
                 dtype: torch.dtype, policy, heavy, recent, softmax_scale: float = 0.0,
                 keep_ids: Sequence[int] = (), vocab: int = 0, proj: Optional[torch.Tensor] = None,
                 history=None, special_ids=None, punct_ids=None, profile_rows: int = 0,
                 profile_threshold: float = 0.0, cache_bits: int = 0, device="cuda"):
        self.layers, self.batch, self.heads, self.head_dim = layers, batch, heads, head_dim
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.max_context, self.dtype, self.device = max_context, dtype, dev
        self.cfg, self._keep = make_config(layers, batch, heads, head_dim, max_context, dtype, policy, heavy,
                                           recent, softmax_scale, keep_ids, vocab, proj, history, special_ids,
                                           punct_ids, profile_rows, profile_threshold, cache_bits)
        self.cache_bits = cache_bits
        self.workspace_bytes = kvevict_workspace_size(self.cfg)
        self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.device)
        self.handle = kvevict_create(self.cfg, self.workspace)

    def close(self) -> None:
        if getattr(self, "handle", None) is not None:
            kvevict_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def capacity(self, layer: int) -> int:
        return kvevict_capacity(self.handle, layer)

    def position(self, layer: int) -> int:
        return kvevict_position(self.handle, layer)

    def _tensor(self, t, shape, dtype, name):
        if t is None:
            return None
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != self.device or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {self.device}, got "
                             f"{t.dtype} {tuple(t.shape)} on {t.device} (contiguous={t.is_contiguous()})")
        return t

    def prefill(self, layer: int, q, k, v, token_ids=None, out=None, stream=None) -> None:
        P = q.shape[2]
        shp = (self.batch, self.heads, P, self.head_dim)
        q, k, v = (self._tensor(x, shp, self.dtype, n) for x, n in ((q, "q"), (k, "k"), (v, "v")))
        token_ids = self._tensor(token_ids, (self.batch, P), torch.int32, "token_ids")
        out = self._tensor(out, shp, torch.float32, "out")
        kvevict_prefill(self.handle, layer, P, q, k, v, token_ids, out, stream)

    def decode_step(self, layer: int, q, k, v, token_ids=None, out=None, evicted=None, stream=None,
                    noalloc: bool = False):
        """One decode step; noalloc=True calls kvevict_decode_step_noalloc (no
        workspace scratch: the library's static per-GPU array instead)."""
        shp = (self.batch, self.heads, self.head_dim)
        q, k, v = (self._tensor(x, shp, self.dtype, n) for x, n in ((q, "q"), (k, "k"), (v, "v")))
        token_ids = self._tensor(token_ids, (self.batch,), torch.int32, "token_ids")
        if out is None:
            out = torch.empty(shp, dtype=torch.float32, device=self.device)
        out = self._tensor(out, shp, torch.float32, "out")
        evicted = self._tensor(evicted, (self.batch, self.heads), torch.int32, "evicted")
        fn = kvevict_decode_step_noalloc if noalloc else kvevict_decode_step
        fn(self.handle, layer, q, k, v, token_ids, out, evicted, stream)
        return out

    def unit_policies(self, layer: int, stream=None) -> torch.Tensor:
        """[batch, heads] int32: the composite each profiled unit chose (0 for other policies)."""
        out = torch.empty((self.batch, self.heads), dtype=torch.int32, device=self.device)
        kvevict_unit_policies(self.handle, layer, out, stream)
        return out

    def cache_rows(self, layer: int, stream=None):
        """Slot contents of one layer: (k, v, k_scale, v_scale).  Rows in the
        storage dtype [batch, heads, cap, d] with null scales, or for 4-bit
        slots uint8 codes [batch, heads, cap, d / 2] (element 2b in the low
        nibble of byte b, stored as code + 8) and float32 scales
        [batch, heads, cap, d / 32]."""
        cap, d = self.capacity(layer), self.head_dim
        if self.cache_bits == 4:
            k = torch.empty((self.batch, self.heads, cap, d // 2), dtype=torch.uint8, device=self.device)
            v = torch.empty_like(k)
            ks = torch.empty((self.batch, self.heads, cap, d // 32), dtype=torch.float32, device=self.device)
            vs = torch.empty_like(ks)
        else:
            k = torch.empty((self.batch, self.heads, cap, d), dtype=self.dtype, device=self.device)
            v = torch.empty_like(k)
            ks = vs = None
        kvevict_cache_rows(self.handle, layer, k, v, ks, vs, stream)
        return k, v, ks, vs

    def kept_indices(self, layer: int, with_scores: bool = True, stream=None):
        cap = self.capacity(layer)
        pos = torch.empty((self.batch, self.heads, cap), dtype=torch.int32, device=self.device)
        cnt = torch.empty((self.batch, self.heads), dtype=torch.int32, device=self.device)
        sc = torch.empty((self.batch, self.heads, cap), dtype=torch.float64, device=self.device) if with_scores else None
        kvevict_kept_indices(self.handle, layer, pos, cnt, sc, stream)
        return pos, cnt, sc
