"""GPU parity at the library's size limits, in its default launch
configuration: the largest context (max_context = 32,768 positions), and the
largest HashEvict budgets (16,384 slots with 16- and 32-bit sketches, 12,288
with 64-bit ones, the most the prompt replay keeps in LDS).

The mixed-policy layer holds one head of each FastGen policy; its FULL head's
slot stride is the whole context, so the split decode grows its chunk until a
unit's chunks fit the combine kernel (768 slots, 43 chunks), and its
frequency + local head runs the prompt scoring and the radix selection over a
32,760-token prompt.  Every unit is replayed against the float64 oracle in
lockstep and checked for the properties that hold at any size."""

import numpy as np
import pytest

from tests import harness
from workloads import configs
from workloads.configs import FULL, H2O, LOCAL, SPECIAL
from workloads.generate import generate_layer

pytestmark = pytest.mark.gpu

MAX_CONTEXT = 32768
STEPS = 8


def run_all_units(w):
    print(f"\n[maxsize] {w.name} B={w.batch} H={w.heads} P={w.prompt} T={w.steps} "
          f"context={w.context} bits={w.sketch_bits}", flush=True)
    inp = generate_layer(w, 0, "cpu", 0)
    kv = harness.make_cache(w, inp, max_context=MAX_CONTEXT)
    r = harness.run_layer(kv, inp.to("cuda"))
    kv.close()
    bad = harness.check_invariants(w, r, w.prompt)
    assert not bad, bad[:10]
    print("[maxsize] invariants ok; oracle on every unit", flush=True)
    rep = harness.check_all(w, inp, r)
    print(f"[maxsize] decisions={rep.decisions} adopted={rep.adopted} max_out={rep.max_out_rel:.2e} "
          f"max_S={rep.max_score_rel:.2e} min_gap={rep.min_gap:.2e}", flush=True)
    assert rep.ok, rep.failures[:10]
    return r


def test_mixed_policy_layer_at_max_context():
    w = configs.scaled("llama65b_fastgen", batch=1, heads=4, prompt=MAX_CONTEXT - STEPS, steps=STEPS)
    pol = w.policy_table(0)[0]
    assert sorted(pol) == sorted([FULL, LOCAL, SPECIAL, H2O])
    r = run_all_units(w)
    h_full = pol.index(FULL)
    # the FULL head holds every position once the last step is in
    assert int(r.final_cnt[0, h_full]) == MAX_CONTEXT


@pytest.mark.parametrize("bits,budget", [(16, 16384), (32, 16384), (64, 12288)])
def test_hash_at_max_budget(bits, budget):
    w = configs.scaled("hashevict_lsh", batch=1, heads=2, prompt=MAX_CONTEXT - STEPS, steps=STEPS,
                       hash_budget=budget, sketch_bits=bits)
    r = run_all_units(w)
    assert (r.final_cnt == budget).all()


def test_q4_hash_at_max_budget():
    """4-bit slots at the largest HashEvict budget: the replay's quantising
    gather of 16,384 rows and the split decode over 4-bit chunks."""
    w = configs.scaled("hashevict_lsh_q4", batch=1, heads=2, prompt=MAX_CONTEXT - STEPS, steps=STEPS,
                       hash_budget=16384)
    assert w.cache_bits == 4
    r = run_all_units(w)
    assert (r.final_cnt == 16384).all()


def test_q4_h2o_at_max_context():
    """4-bit slots on H2O heads with a 32,760-token prompt and a 2,048 + 2,048
    slot budget (the split decode over 4-bit rows, the quantising gather of
    the selected prompt rows)."""
    w = configs.scaled("opt30b_decode_h2o_q4", layers=1, batch=1, heads=2, prompt=MAX_CONTEXT - STEPS,
                       steps=STEPS, heavy=2048, recent=2048)
    assert w.cache_bits == 4
    r = run_all_units(w)
    assert (r.final_cnt == 4096).all()


def test_persist_at_max_context():
    """Persistence counts with a 32,760-token prompt (pivotal bits of the
    last 64 prompt rows, popcount ranking over 28,664 candidates) and
    2,048 + 2,048 slots (split decode)."""
    w = configs.scaled("opt30b_decode_persist", layers=1, batch=1, heads=2, prompt=MAX_CONTEXT - STEPS,
                       steps=STEPS, heavy=2048, recent=2048)
    r = run_all_units(w)
    assert (r.final_cnt == 4096).all()


def test_profiled_fastgen_at_max_context():
    """FastGen profiling with a 32,760-token prompt: one head of each of the
    five attention kinds, each unit's composite chosen from the last 64
    prompt rows, caches whose stride is the whole 32,768-position context
    (the grown split chunk)."""
    w = configs.scaled("llama65b_fastgen_profiled", batch=1, heads=5, prompt=MAX_CONTEXT - STEPS, steps=STEPS)
    run_all_units(w)
