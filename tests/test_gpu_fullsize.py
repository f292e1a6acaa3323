"""GPU parity at full workload sizes, in the launch configuration the bench
uses (one layer of each workload's real shape; configs 4 and 5 take the split
decode, configs 2 and 3 the fused one).

Every unit is checked for the properties that hold at any size (budget,
recent window, unique in-range positions, finite outputs); a seeded sample of
units, always including the first and the last, is replayed against the
float64 oracle in lockstep."""

import numpy as np
import pytest
import torch

from tests import harness
from workloads import configs
from workloads.configs import FULL, H2O, HASH, LOCAL, SPECIAL
from oracle import attention, lockstep
from workloads.generate import generate_layer, unit_sequence

pytestmark = pytest.mark.gpu


def sample_units(w, n, seed=0, heads_of=None):
    rng = np.random.default_rng(seed)
    units = {(0, 0), (w.batch - 1, w.heads - 1)}
    if heads_of is not None:                      # one unit per listed head kind
        pol = w.policy_table(0)[0]
        for kind in heads_of:
            h = pol.index(kind)
            units.add((int(rng.integers(w.batch)), h))
    while len(units) < n:
        units.add((int(rng.integers(w.batch)), int(rng.integers(w.heads))))
    return sorted(units)


def run_full(name, n_sample, heads_of=None):
    w = configs.get(name)
    print(f"\n[fullsize] {name}: units={w.units_per_layer} P={w.prompt} T={w.steps}", flush=True)
    inp = generate_layer(w, 0, "cuda", 0)
    kv = harness.make_cache(w, inp)
    r = harness.run_layer(kv, inp)
    kv.close()
    bad = harness.check_invariants(w, r, w.prompt)
    assert not bad, bad[:10]
    units = sample_units(w, n_sample, heads_of=heads_of)
    print(f"[fullsize] invariants ok on all units; oracle on {units}", flush=True)
    rep = harness.check_all(w, inp, r, units)
    print(f"[fullsize] decisions={rep.decisions} adopted={rep.adopted} max_out={rep.max_out_rel:.2e} "
          f"max_S={rep.max_score_rel:.2e} min_gap={rep.min_gap:.2e}", flush=True)
    assert rep.ok, rep.failures[:10]
    return rep


def test_opt6_7b_layer_full_size():
    run_full("opt6.7b_layer_h2o", 12)


def test_opt30b_layer_full_size():
    run_full("opt30b_decode_h2o", 8)


def test_opt30b_persist_layer_full_size():
    rep = run_full("opt30b_decode_persist", 6)
    assert rep.decisions == 6 * 256


def test_llama65b_fastgen_profiled_full_size():
    rep = run_full("llama65b_fastgen_profiled", 6)
    assert rep.decisions > 0


def test_llama65b_fastgen_full_size():
    run_full("llama65b_fastgen", 8, heads_of=[FULL, H2O, LOCAL, SPECIAL])


def test_hashevict_full_size():
    rep = run_full("hashevict_lsh", 4)
    assert rep.decisions == 4 * 1024


@pytest.mark.parametrize("name", ["hashevict_lsh", "opt30b_decode_h2o"])
def test_prompt_output_full_size(name):
    """The optional prompt output at a full prompt (all units of one layer in
    one launch): sampled rows of sampled units against the float64 oracle,
    every row finite."""
    w = configs.get(name)
    print(f"\n[fullsize] {name}: prompt output, units={w.units_per_layer} P={w.prompt}", flush=True)
    inp = generate_layer(w, 0, "cuda", 1)
    kv = harness.make_cache(w, inp)
    po = torch.empty((w.batch, w.heads, w.prompt, w.head_dim), dtype=torch.float32, device="cuda")
    ids = inp.ids[:, :w.prompt].contiguous() if inp.ids is not None else None
    kv.prefill(0, inp.prompt_q, inp.prompt_k, inp.prompt_v, ids, po)
    torch.cuda.synchronize()
    kv.close()
    assert bool(torch.isfinite(po).all())
    rng = np.random.default_rng(0)
    inp_cpu = inp.to("cpu")
    P, scale = w.prompt, 1.0 / np.sqrt(w.head_dim)
    worst = 0.0
    for b, h in sample_units(w, 3):
        Q, K, V = unit_sequence(inp_cpu, b, h)
        rows = sorted({0, 1, 63, 64, 127, 128, P - 2, P - 1, *rng.integers(0, P, 8).tolist()})
        got = po[b, h, rows].cpu().double().numpy()
        for n, i in enumerate(rows):
            _, ref = attention.attend(Q[i], K[:i + 1], V[:i + 1], scale)
            e = np.max(np.abs(got[n] - ref)) / max(np.max(np.abs(ref)), 1e-30)
            worst = max(worst, e)
            assert e <= lockstep.OUT_RTOL, (b, h, i, e)
    print(f"[fullsize] prompt output max rel err {worst:.2e}", flush=True)


def test_opt30b_q4_layer_full_size():
    """4-bit slots at the OPT-30B shape: lockstep on sampled units against the
    oracle with quantised cache rows."""
    rep = run_full("opt30b_decode_h2o_q4", 6)
    assert rep.decisions == 6 * 256


def test_hashevict_q4_full_size():
    rep = run_full("hashevict_lsh_q4", 4)
    assert rep.decisions == 4 * 1024
