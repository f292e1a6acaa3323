"""GPU parity: the HIP path through the C ABI against the float64 oracle, in
lockstep (kept sets exact up to the 1e-6 near-tie band, scores within 1e-5,
outputs within 2e-3 of the max output element).

Sizes are scaled-down versions of the five workloads that still span several
tiles and a ragged tail; full-size launches are checked on sampled units in
test_gpu_fullsize.py."""

import dataclasses

import numpy as np
import pytest
import torch

from tests import harness
from workloads import configs
from workloads.configs import ADAPTIVE, FULL, H2O, HASH, LOCAL, PERSIST, SPECIAL
from workloads.generate import generate_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["fused", "split"])
def decode_path(request, monkeypatch):
    """Runs a test with the one-workgroup-per-unit decode and again with the
    split decode forced at small sizes (chunks of 32 slots)."""
    if request.param == "split":
        monkeypatch.setenv("KVEVICT_SPLIT_ABOVE", "0")
        monkeypatch.setenv("KVEVICT_SPLIT_CHUNK", "32")
    return request.param


def run_and_check(w, policy=None, heavy=None, recent=None, prompt_out=False, seed=0, units=None,
                  history=None):
    import os
    print(f"\n[parity] split_above={os.environ.get('KVEVICT_SPLIT_ABOVE', '-')} {w.name} B={w.batch} H={w.heads} d={w.head_dim} {w.dtype} P={w.prompt} "
          f"T={w.steps} seed={seed}", flush=True)
    inp = generate_layer(w, 0, "cpu", seed)
    kv = harness.make_cache(w, inp, policy, heavy, recent, history=history)
    r = harness.run_layer(kv, inp.to("cuda"), want_prompt_out=prompt_out)
    rep = harness.check_all(w, inp, r, units, policy=policy, heavy=heavy, recent=recent, history=history)
    print(f"[parity] decisions={rep.decisions} adopted={rep.adopted} max_out={rep.max_out_rel:.2e} "
          f"max_prompt_out={rep.max_prompt_out_rel:.2e} max_S={rep.max_score_rel:.2e} "
          f"min_gap={rep.min_gap:.2e}", flush=True)
    assert rep.ok, rep.failures[:10]
    bad = harness.check_invariants(w, r, inp.prompt_q.shape[2], policy, heavy, recent, history)
    assert not bad, bad[:10]
    kv.close()
    return rep, r


def test_tiny_h2o_full_size(decode_path):
    rep, _ = run_and_check(configs.get("tiny_h2o"), prompt_out=True)
    assert rep.decisions == 2 * 64


def test_h2o_fp16_scaled(decode_path):
    w = configs.scaled("opt6.7b_layer_h2o", batch=2, heads=4, prompt=300, steps=90)
    assert (w.heavy, w.recent) == (30, 30)
    run_and_check(w, prompt_out=True)


def test_h2o_bf16_scaled(decode_path):
    w = configs.scaled("opt30b_decode_h2o", batch=2, heads=3, prompt=700, steps=60)
    run_and_check(w)


def test_h2o_fp32_d128():
    w = dataclasses.replace(configs.scaled("opt6.7b_layer_h2o", batch=1, heads=3, prompt=150, steps=40),
                            dtype="f32")
    run_and_check(w, prompt_out=True)


def test_fastgen_scaled(decode_path):
    w = configs.scaled("llama65b_fastgen", batch=2, heads=8, prompt=500, steps=60)
    assert (w.local_window, w.freq_heavy) == (125, 50)
    run_and_check(w, prompt_out=True)


def test_hash_scaled(decode_path):
    w = configs.scaled("hashevict_lsh", batch=2, heads=4, prompt=600, steps=80)
    assert w.hash_budget == 300
    rep, _ = run_and_check(w, prompt_out=True)
    assert rep.decisions == 8 * 80


@pytest.mark.parametrize("dtype,P", [("f16", 200), ("bf16", 129), ("bf16", 64)])
def test_prompt_out_d64_16bit(dtype, P):
    """Matrix-core prompt output at head_dim 64: a ragged prompt, one just
    past a 128-query block, and exactly one 64-key tile."""
    w = dataclasses.replace(configs.scaled("tiny_h2o", prompt=P, steps=20, batch=2), dtype=dtype)
    rep, _ = run_and_check(w, prompt_out=True)
    assert rep.max_prompt_out_rel > 0


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prompt_out_one_token(dtype):
    w = dataclasses.replace(configs.scaled("opt6.7b_layer_h2o", batch=1, heads=2, prompt=1, steps=30), dtype=dtype)
    run_and_check(w, policy=[H2O] * 2, heavy=[4] * 2, recent=[4] * 2, prompt_out=True)


def test_budget_covering_context_is_full_attention(decode_path):
    """heavy + recent >= P + T: nothing is evicted; outputs equal causal attention."""
    w = configs.scaled("opt30b_decode_h2o", batch=1, heads=2, prompt=100, steps=40)
    N = w.context
    rep, r = run_and_check(w, policy=[H2O] * 2, heavy=[N - 10] * 2, recent=[10] * 2, prompt_out=True)
    assert (r.evicted == -1).all()


@pytest.mark.parametrize("P,T,hh,rc", [(1, 30, 4, 4), (5, 40, 8, 8), (90, 30, 12, 0), (90, 30, 0, 12),
                                       (64, 64, 16, 16), (257, 20, 100, 27)])
def test_h2o_edge_shapes(P, T, hh, rc, decode_path):
    """Prompt of one token, prompt shorter than the budget (the cache grows),
    no recent window (the new token may be evicted at once), no heavy part,
    tile-aligned and ragged prompts."""
    w = configs.scaled("opt6.7b_layer_h2o", batch=1, heads=2, prompt=P, steps=T)
    run_and_check(w, policy=[H2O] * 2, heavy=[hh] * 2, recent=[rc] * 2)


def test_special_without_kept_prompt_tokens(decode_path):
    w = configs.scaled("llama65b_fastgen", batch=1, heads=4, prompt=20, steps=30)
    w = dataclasses.replace(w, special_ids=(31990,), punct_ids=(31991,))   # (almost) never drawn
    run_and_check(w, policy=[SPECIAL, FULL, LOCAL, SPECIAL], heavy=[0] * 4, recent=[0, 0, 7, 0])


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_hash_fp16_fp32_rows(dtype, decode_path):
    """HashEvict with fp16 and fp32 rows: their sketches take the float64
    path (bf16 rows take the matrix cores), then the register replay."""
    w = dataclasses.replace(configs.scaled("hashevict_lsh", batch=1, heads=3, prompt=400, steps=40), dtype=dtype)
    assert w.hash_budget == 200
    rep, _ = run_and_check(w)
    assert rep.decisions == 3 * 40


def test_hash_prompt_shorter_than_budget(decode_path):
    w = configs.scaled("hashevict_lsh", batch=1, heads=2, prompt=50, steps=40)
    run_and_check(w, policy=[HASH] * 2, heavy=[70] * 2, recent=[0] * 2)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_h2o_bf16_more_seeds(seed, decode_path):
    w = configs.scaled("opt30b_decode_h2o", batch=2, heads=2, prompt=333, steps=50)
    run_and_check(w, seed=seed)


def test_deterministic_across_runs(decode_path):
    w = configs.scaled("opt6.7b_layer_h2o", batch=2, heads=2, prompt=200, steps=30)
    inp = generate_layer(w, 0, "cpu", 3).to("cuda")
    runs = []
    for _ in range(2):
        kv = harness.make_cache(w, inp)
        runs.append(harness.run_layer(kv, inp))
        kv.close()
    a, b = runs
    for f in ("out", "evicted", "final_pos", "final_S", "prefill_S"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


# ---- persistence counts (Scissorhands reading)

def test_persist_bf16_scaled(decode_path):
    w = configs.scaled("opt30b_decode_persist", batch=2, heads=3, prompt=700, steps=80)
    assert (w.heavy, w.recent, w.history_window) == (70, 70, 64)
    rep, _ = run_and_check(w)
    assert rep.decisions == 6 * 80


def test_persist_fp16_d64_and_mixed_windows(decode_path):
    """d = 64 fp16, windows 1, 17, 64 and one H2O head in the same layer."""
    w = dataclasses.replace(configs.scaled("opt30b_decode_persist", batch=2, heads=4, prompt=300, steps=60),
                            dtype="f16", head_dim=64)
    run_and_check(w, policy=[PERSIST, PERSIST, H2O, PERSIST], heavy=[30, 20, 30, 10], recent=[30, 5, 30, 40],
                  history=[1, 17, 0, 64])


def test_persist_fp32(decode_path):
    w = dataclasses.replace(configs.scaled("opt30b_decode_persist", batch=1, heads=3, prompt=150, steps=40),
                            dtype="f32")
    run_and_check(w, prompt_out=True, history=[64, 9, 33])


@pytest.mark.parametrize("P,T,hh,rc,win", [(1, 30, 4, 4, 64), (5, 40, 8, 8, 3), (90, 30, 12, 0, 64),
                                           (90, 30, 0, 12, 10), (64, 64, 16, 16, 64), (257, 20, 100, 27, 40),
                                           (130, 40, 20, 20, 64)])
def test_persist_edge_shapes(P, T, hh, rc, win, decode_path):
    """One-token prompt, prompt shorter than the budget, no recent window (the
    new token may leave at once), no heavy part, tile-aligned and ragged
    prompts, a window reaching across a 128-query block boundary."""
    w = configs.scaled("opt30b_decode_persist", batch=1, heads=2, prompt=P, steps=T)
    run_and_check(w, policy=[PERSIST] * 2, heavy=[hh] * 2, recent=[rc] * 2, history=[win] * 2)


def test_persist_identical_keys_is_a_sliding_window(decode_path):
    """Every key equal: every decode weight is exactly 1 / |A| (pivotal at
    every step), so once the cache is full the oldest candidate leaves at each
    step.  The prompt fits the budget and the 4-step window has forgotten the
    prompt rows (whose weights are uniform only up to rounding) before the
    first eviction."""
    P, T, hh, rc, win = 60, 60, 8, 70, 4
    B = hh + rc
    w = configs.scaled("opt30b_decode_persist", batch=1, heads=2, prompt=P, steps=T)
    inp = generate_layer(w, 0, "cpu", 0)
    inp.prompt_k[:] = inp.prompt_k[:, :, :1]
    inp.dec_k[:] = inp.prompt_k[:, :, 0].unsqueeze(0)
    kv = harness.make_cache(w, inp, policy=[PERSIST] * 2, heavy=[hh] * 2, recent=[rc] * 2, history=[win] * 2)
    r = harness.run_layer(kv, inp.to("cuda"))
    kv.close()
    for h in range(2):
        assert sorted(r.prefill_pos[0, h, :P].tolist()) == list(range(P))
        assert r.evicted[:, 0, h].tolist() == [P + s - B if P + s >= B else -1 for s in range(T)]
        assert sorted(r.final_pos[0, h, :B].tolist()) == list(range(P + T - B, P + T))
        bits = np.ascontiguousarray(r.final_S[0, h, :B]).view(np.uint64)
        assert (bits == np.uint64(15)).sum() == B - 3    # all but the three newest hold 4 set bits


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_logit_jump_after_first_tile(dtype):
    """A key far past the first 64-key tile whose logit with every later
    query exceeds everything before it by ~200 (log2 units): the row pass must
    leave its running offset and refold that tile at the new maximum."""
    w = dataclasses.replace(configs.scaled("opt30b_decode_h2o", batch=1, heads=2, prompt=300, steps=20),
                            dtype=dtype)
    inp = generate_layer(w, 0, "cpu", 5)
    u = torch.zeros(w.head_dim)
    u[3] = 1.0
    amp = 40.0 if dtype == "bf16" else 30.0          # |s| / sqrt(d) * log2(e): 204 (bf16), 115 (f16)
    inp.prompt_k[0, :, 150] = (amp * u).to(inp.prompt_k.dtype)
    inp.prompt_q[0, :, 151:] += (amp * u).to(inp.prompt_q.dtype)
    rep, _ = run_and_check(w)
    assert rep.ok


# ---- FastGen profiling (adaptive composites)

def test_adaptive_bf16_scaled(decode_path):
    """Ten heads of the five attention kinds, two sequences: every composite
    is chosen somewhere; lockstep against the oracle's profile and trajectory."""
    w = configs.scaled("llama65b_fastgen_profiled", batch=2, heads=10, prompt=600, steps=60)
    rep, r = run_and_check(w)
    assert set(np.unique(r.choice).tolist()) == {1, 2, 3, 4, 5}, r.choice


def test_adaptive_fp16_d64_and_short_prompt(decode_path):
    w = dataclasses.replace(configs.scaled("llama65b_fastgen_profiled", batch=1, heads=5, prompt=40, steps=50),
                            dtype="f16", head_dim=64)
    run_and_check(w)


def test_adaptive_fp32_with_prompt_out():
    w = dataclasses.replace(configs.scaled("llama65b_fastgen_profiled", batch=1, heads=5, prompt=200, steps=30),
                            dtype="f32")
    run_and_check(w, prompt_out=True)


@pytest.mark.parametrize("thr", [0.0, 2.0])
def test_adaptive_threshold_extremes(thr, decode_path):
    """Threshold 0: every unit takes the special-token composite; above 1:
    every unit keeps the full cache."""
    w = dataclasses.replace(configs.scaled("llama65b_fastgen_profiled", batch=1, heads=5, prompt=300, steps=40),
                            profile_threshold=thr)
    rep, r = run_and_check(w)
    assert (r.choice == (1 if thr == 0.0 else 5)).all()


@pytest.mark.parametrize("bits", [16, 64])
def test_hash_sketch_widths(bits, decode_path):
    """16- and 64-bit sketches (32 is the workload's width): bit-exact
    decisions against the oracle, including a budget above a 64-bit word's
    vector-load multiple and a unit stride that is not."""
    w = dataclasses.replace(configs.scaled("hashevict_lsh", batch=2, heads=3, prompt=500, steps=70),
                            sketch_bits=bits)
    assert w.hash_budget == 250
    rep, _ = run_and_check(w)
    assert rep.decisions == 6 * 70


@pytest.mark.parametrize("budget", [1, 3, 64, 255, 257, 1024, 1027, 4096, 4097])
def test_hash_replay_budgets(budget):
    """Prompt replay and decode replacement at budgets that leave whole waves
    of the workgroup without a slot (1, 3, 64), that are not a multiple of the
    four-slot scan rounds or of the 256 threads (255, 257, 1027), and at the
    edges of the register replay's two sizes (1,024 and 4,096 slots: every
    register group full; 4,097: the replay with slot state in LDS):
    bit-exact decisions against the oracle, every prompt position past the
    budget replayed."""
    w = configs.scaled("hashevict_lsh", batch=1, heads=2, prompt=budget + 300, steps=30)
    rep, r = run_and_check(w, policy=[HASH] * 2, heavy=[budget] * 2, recent=[0] * 2)
    assert (r.final_cnt == budget).all()
