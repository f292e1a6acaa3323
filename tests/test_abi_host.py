"""The C ABI library loads, exports every symbol the header declares, and
validates arguments on the host (CPU only: no call here reaches the GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

from budgeted_decode_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "kvevict.h")).read()
    return sorted(set(re.findall(r"\b(kvevict_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = binding.load_library()
    names = header_functions()
    assert len(names) == 14
    assert set(names) == set(binding.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def cfg(**over):
    base = dict(layers=1, batch=2, heads=3, head_dim=128, max_context=100, dtype=torch.bfloat16,
                policy=[1, 1, 1], heavy=[10, 10, 10], recent=[5, 5, 5])
    base.update(over)
    return binding.make_config(**base)


def status_of(c):
    n = ctypes.c_size_t(0)
    return binding.load_library().kvevict_workspace_size(ctypes.byref(c), ctypes.byref(n)), n.value


def test_workspace_size_accepts_valid_configs_and_scales():
    c, keep = cfg()
    s, n1 = status_of(c)
    assert s == binding.KVE_OK and n1 > 0
    c, keep = cfg(max_context=1000)
    s, n2 = status_of(c)
    assert s == binding.KVE_OK and n2 > n1


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=96), binding.KVE_EUNSUPPORTED),
    (dict(max_context=0), binding.KVE_EUNSUPPORTED),
    (dict(max_context=40000), binding.KVE_EUNSUPPORTED),
    (dict(policy=[7, 1, 1]), binding.KVE_EINVAL),
    (dict(heavy=[0, 10, 10], recent=[0, 5, 5]), binding.KVE_EINVAL),
    (dict(heavy=[-1, 10, 10]), binding.KVE_EINVAL),
    (dict(heavy=[90, 10, 10], recent=[20, 5, 5]), binding.KVE_EINVAL),
    (dict(policy=[2, 1, 1], heavy=[3, 10, 10]), binding.KVE_EINVAL),
    (dict(policy=[0, 1, 1], heavy=[0, 10, 10], recent=[1, 5, 5]), binding.KVE_EINVAL),
    (dict(policy=[3, 1, 1], heavy=[0, 10, 10], recent=[0, 5, 5]), binding.KVE_EINVAL),
    (dict(policy=[4, 1, 1], heavy=[50, 10, 10], recent=[0, 5, 5]), binding.KVE_EUNSUPPORTED),
    (dict(layers=0), binding.KVE_EINVAL),
    (dict(softmax_scale=float("nan")), binding.KVE_EINVAL),
])
def test_workspace_size_rejects_bad_configs(over, status):
    c, keep = cfg(**over)
    s, _ = status_of(c)
    assert s == status
    assert binding.load_library().kvevict_last_error().decode() != ""


def test_special_and_hash_need_their_tables():
    c, keep = cfg(policy=[3, 1, 1], heavy=[0, 10, 10], recent=[0, 5, 5], keep_ids=[0, 1], vocab=100)
    assert status_of(c)[0] == binding.KVE_OK
    proj = torch.zeros((128, 32), dtype=torch.bfloat16)
    c, keep = cfg(policy=[4, 1, 1], heavy=[50, 10, 10], recent=[0, 5, 5], proj=proj)
    assert status_of(c)[0] == binding.KVE_OK


def test_create_rejects_small_or_misaligned_workspace_without_touching_it():
    lib = binding.load_library()
    c, keep = cfg()
    n = ctypes.c_size_t(0)
    lib.kvevict_workspace_size(ctypes.byref(c), ctypes.byref(n))
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 40)          # never dereferenced: checks fail first
    assert lib.kvevict_create(ctypes.byref(c), fake, n.value - 1, ctypes.byref(h)) == binding.KVE_ENOMEM
    assert lib.kvevict_create(ctypes.byref(c), ctypes.c_void_p((1 << 40) + 8), n.value,
                              ctypes.byref(h)) == binding.KVE_EINVAL
    assert lib.kvevict_create(ctypes.byref(c), None, n.value, ctypes.byref(h)) == binding.KVE_EINVAL
    assert h.value is None


def test_calls_on_a_null_handle_fail_cleanly():
    lib = binding.load_library()
    assert lib.kvevict_prefill(None, 0, 10, None, None, None, None, None, None) == binding.KVE_EINVAL
    assert lib.kvevict_decode_step(None, 0, None, None, None, None, None, None, None) == binding.KVE_EINVAL
    assert lib.kvevict_kept_indices(None, 0, None, None, None, None) == binding.KVE_EINVAL
    assert lib.kvevict_destroy(None) == binding.KVE_EINVAL
    assert lib.kvevict_capacity(None, 0) == -1 and lib.kvevict_position(None, 0) == -1
    for s in range(6):
        assert lib.kvevict_status_string(s)


@pytest.mark.parametrize("history,status", [
    (None, binding.KVE_EINVAL),                 # PERSIST heads need the table
    ([0, 0, 0], binding.KVE_EINVAL),            # window < 1
    ([65, 1, 1], binding.KVE_EINVAL),           # window > 64
    ([64, 0, 0], binding.KVE_OK),               # other heads' entries are ignored
    ([1, 7, 9], binding.KVE_OK),
])
def test_persist_needs_a_history_window(history, status):
    c, keep = cfg(policy=[5, 1, 1], history=history)
    assert status_of(c)[0] == status


def test_persist_capacity_is_heavy_plus_recent():
    a, ka = cfg(policy=[5, 5, 5], history=[8, 8, 8])
    b, kb = cfg()
    assert status_of(a) == status_of(b)   # same slots and workspace as the H2O table


@pytest.mark.parametrize("over,status", [
    (dict(), binding.KVE_OK),
    (dict(profile_rows=0), binding.KVE_EINVAL),
    (dict(profile_threshold=float("inf")), binding.KVE_EINVAL),
    (dict(heavy=[-1, 10, 10]), binding.KVE_EINVAL),
    (dict(heavy=[5, 10, 10], recent=[4, 5, 5], policy=[6, 6, 1]), binding.KVE_EUNSUPPORTED),  # mixed budgets
])
def test_adaptive_configs(over, status):
    base = dict(policy=[6, 6, 1], heavy=[10, 10, 10], recent=[5, 5, 5], special_ids=[0, 1], punct_ids=[2],
                vocab=100, profile_rows=16, profile_threshold=0.9)
    base.update(over)
    c, keep = cfg(**base)
    assert status_of(c)[0] == status


def test_adaptive_needs_its_id_sets():
    c, keep = cfg(policy=[6, 1, 1], vocab=100, keep_ids=[0])
    assert status_of(c)[0] == binding.KVE_EINVAL


@pytest.mark.parametrize("bits,budget,status", [(16, 50, binding.KVE_OK), (64, 50, binding.KVE_OK),
                                                (48, 50, binding.KVE_EUNSUPPORTED)])
def test_sketch_widths(bits, budget, status):
    proj = torch.zeros((128, bits), dtype=torch.bfloat16)
    c, keep = cfg(policy=[4, 1, 1], heavy=[budget, 10, 10], recent=[0, 5, 5], proj=proj)
    assert status_of(c)[0] == status


def test_64_bit_sketches_cap_the_budget():
    proj = torch.zeros((128, 64), dtype=torch.bfloat16)
    c, keep = cfg(policy=[4, 1, 1], heavy=[13000, 10, 10], recent=[0, 5, 5], proj=proj, max_context=20000)
    assert status_of(c)[0] == binding.KVE_EINVAL
    c, keep = cfg(policy=[4, 1, 1], heavy=[12288, 10, 10], recent=[0, 5, 5], proj=proj, max_context=20000)
    assert status_of(c)[0] == binding.KVE_OK


@pytest.mark.parametrize("over,status", [
    (dict(cache_bits=4), binding.KVE_OK),
    (dict(cache_bits=4, policy=[5, 1, 5], history=[8, 8, 8]), binding.KVE_OK),
    (dict(cache_bits=4, head_dim=64), binding.KVE_OK),
    (dict(cache_bits=4, dtype=torch.float32), binding.KVE_OK),
    (dict(cache_bits=8), binding.KVE_EUNSUPPORTED),
    (dict(cache_bits=4, policy=[2, 1, 1], heavy=[0, 10, 10], recent=[5, 5, 5]), binding.KVE_EUNSUPPORTED),
    (dict(cache_bits=4, policy=[0, 1, 1], heavy=[0, 10, 10], recent=[0, 5, 5]), binding.KVE_EUNSUPPORTED),
    (dict(cache_bits=4, policy=[4, 1, 1], heavy=[50, 10, 10], recent=[0, 5, 5],
          proj=torch.zeros((128, 32), dtype=torch.bfloat16)), binding.KVE_OK),
])
def test_four_bit_slots_configs(over, status):
    c, keep = cfg(**over)
    assert status_of(c)[0] == status


def test_four_bit_slots_shrink_the_workspace():
    # per slot: d / 2 code bytes and d / 32 float scales for K and for V
    # (160 bytes at d 128) in place of 2 * d * 2 bytes of bf16 rows (512)
    # (a fused-decode size: no split scratch, whose chunking differs with the format)
    big = dict(max_context=4096, heavy=[500, 500, 500], recent=[500, 500, 500])
    s16, n16 = status_of(cfg(**big)[0])
    s4, n4 = status_of(cfg(cache_bits=4, **big)[0])
    assert s16 == s4 == binding.KVE_OK
    units, cap = 2 * 3, 1000
    assert abs((n16 - n4) - units * cap * (512 - 160)) < 16 * 256


def test_cache_rows_rejects_a_null_handle():
    lib = binding.load_library()
    assert lib.kvevict_cache_rows(None, 0, None, None, None, None, None) == binding.KVE_EINVAL


def test_mixed_layer_at_max_context_is_accepted():
    """A layer mixing a FULL head (stride = the whole context) with other
    policies at max_context 32768: the split decode's chunk grows until a
    unit's chunks fit the combine kernel, so the layer is accepted."""
    c, keep = cfg(batch=1, heads=4, max_context=32768, policy=[0, 2, 3, 1], heavy=[0, 0, 0, 3276],
                  recent=[0, 8190, 0, 8190], keep_ids=list(range(14)), vocab=32000)
    s, n = status_of(c)
    assert s == binding.KVE_OK, binding.load_library().kvevict_last_error()
    assert n > 0


def test_stream_read_validates_arguments():
    lib = binding.load_library()
    fake = ctypes.c_void_p((1 << 40))
    sink = ctypes.c_void_p((1 << 40) + 4096)
    assert lib.kvevict_stream_read(None, 64, sink, None) == binding.KVE_EINVAL
    assert lib.kvevict_stream_read(fake, 64, None, None) == binding.KVE_EINVAL
    assert lib.kvevict_stream_read(fake, 0, sink, None) == binding.KVE_EINVAL
    assert lib.kvevict_stream_read(fake, 72, sink, None) == binding.KVE_EINVAL          # not a multiple of 16
    assert lib.kvevict_stream_read(ctypes.c_void_p((1 << 40) + 8), 64, sink, None) == binding.KVE_EINVAL


def test_decode_step_noalloc_validates_on_the_host():
    lib = binding.load_library()
    assert lib.kvevict_decode_step_noalloc(None, 0, None, None, None, None, None, None, None) == binding.KVE_EINVAL
