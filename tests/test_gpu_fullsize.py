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
from workloads.generate import generate_layer

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


def test_llama65b_fastgen_full_size():
    run_full("llama65b_fastgen", 8, heads_of=[FULL, H2O, LOCAL, SPECIAL])


def test_hashevict_full_size():
    rep = run_full("hashevict_lsh", 4)
    assert rep.decisions == 4 * 1024
