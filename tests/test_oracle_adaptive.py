"""Pins of FastGen's profiling and composite policies (CPU only).

The composite rule reduces to the separately pinned H2O, special-token and
full-cache oracles in its special cases; the profile has a closed form on
uniform attention (harmonic numbers); the greedy composites are nested.
"""

import numpy as np
import pytest

from oracle import adaptive, fastgen, h2o
from oracle.attention import causal_weights


def rand_case(seed, N, d, vocab=20):
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    ids = rng.integers(0, vocab, N)
    return Q, K, V, ids


@pytest.mark.parametrize("seed", range(3))
def test_no_protected_ids_is_h2o(seed):
    Q, K, V, ids = rand_case(seed, 70, 8)
    comp = adaptive.Composite(frozenset(), 6, 9)
    k0, S0, out, ev, kept, S = adaptive.run_composite(comp, Q, K, V, ids, 40, 0.5)
    tr = h2o.run_unit(Q, K, V, 40, 6, 9, 0.5)
    assert np.array_equal(k0, tr.prefill_kept)
    assert np.array_equal(ev, tr.evicted)
    assert np.array_equal(np.sort(kept), np.sort(tr.final.pos))
    np.testing.assert_allclose(out, tr.out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S0, tr.prefill_scores, rtol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_no_slots_is_the_special_policy(seed):
    Q, K, V, ids = rand_case(10 + seed, 60, 8)
    keep = [0, 3, 7]
    comp = adaptive.Composite(frozenset(keep), 0, 0)
    k0, S0, out, ev, kept, S = adaptive.run_composite(comp, Q, K, V, ids, 30, 0.5)
    tr = fastgen.run_special(Q, K, V, ids, keep, 30, 0.5)
    assert np.array_equal(k0, tr.prefill_kept)
    assert np.array_equal(ev, tr.evicted)
    assert np.array_equal(np.sort(kept), tr.final_kept)
    np.testing.assert_allclose(out, tr.out, rtol=0, atol=1e-12)


def test_full_composite_is_the_full_cache():
    Q, K, V, ids = rand_case(5, 50, 8)
    comp = adaptive.Composite(frozenset(), 0, 0, True)
    k0, S0, out, ev, kept, S = adaptive.run_composite(comp, Q, K, V, ids, 20, 0.5)
    tr = fastgen.run_full(Q, K, V, 20, 0.5)
    assert (ev == -1).all() and np.array_equal(kept, np.arange(50))
    np.testing.assert_allclose(out, tr.out, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_protected_tokens_stay_and_the_rest_keeps_its_budget(seed):
    Q, K, V, ids = rand_case(20 + seed, 90, 8, vocab=6)
    comp = adaptive.Composite(frozenset([0, 1]), 5, 7)
    k0, S0, out, ev, kept, S = adaptive.run_composite(comp, Q, K, V, ids, 40, 0.5)
    prot = [j for j in range(90) if ids[j] in (0, 1)]
    assert set(prot) <= set(kept.tolist())
    assert not set(prot) & set(int(e) for e in ev)
    free = [j for j in kept if ids[j] not in (0, 1)]
    assert len(free) <= 12
    assert set(j for j in range(90 - 7, 90) if ids[j] not in (0, 1)) <= set(kept.tolist())


def test_profile_closed_form_on_uniform_attention():
    """Identical keys: row i gives 1/(i+1) to each key 0..i.  With only
    position 0 special, C1 recovers (H_P - H_{P-R}) / R over the last R rows."""
    P, R, d = 50, 16, 8
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((P, d))
    K = np.tile(rng.standard_normal(d), (P, 1))
    ids = np.full(P, 9)
    ids[0] = 0
    comps = adaptive.composites([0], [1], 4, 6)
    k, rec = adaptive.profile(Q, K, ids, comps, 0.5, R, 2.0)
    H = lambda n: sum(1.0 / i for i in range(1, n + 1))
    assert rec[adaptive.C_SPECIAL] == pytest.approx((H(P) - H(P - R)) / R, rel=1e-12)
    assert k == adaptive.C_FULL                                      # threshold 2 is never reached
    k0, _ = adaptive.profile(Q, K, ids, comps, 0.5, R, 0.0)
    assert k0 == adaptive.C_SPECIAL                                  # threshold 0: the first composite


@pytest.mark.parametrize("seed", range(4))
def test_greedy_composites_are_nested_and_the_choice_is_the_first_reaching_the_threshold(seed):
    P, d = 60, 8
    Q, K, V, ids = rand_case(40 + seed, P, d, vocab=8)
    comps = adaptive.composites([0], [1, 2], 5, 10)
    p = causal_weights(Q, K, 0.5)
    c = p.sum(axis=0)
    sets = {k: set(adaptive.prompt_kept(comps[k], c, ids, P).tolist()) for k in (1, 2, 3, 4)}
    assert sets[1] <= sets[2] <= sets[3]
    _, rec = adaptive.profile(Q, K, ids, comps, 0.5, 20, 2.0)
    assert rec[1] <= rec[2] + 1e-15 <= rec[3] + 2e-15
    for T in (0.0, rec[2], (rec[2] + rec[3]) / 2, rec[4], 1.5):
        k, r2 = adaptive.profile(Q, K, ids, comps, 0.5, 20, T)
        first = next((j for j in (1, 2, 3, 4) if r2[j] >= T), 5) if k != 5 else 5
        assert k == first
        assert all(r2[j] < T for j in r2 if j < k)


def test_dominant_special_token_profiles_as_special():
    """A special-id token that takes almost all of every row's weight: C1
    already recovers nearly everything."""
    P, d = 40, 16
    rng = np.random.default_rng(3)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    Q = 4.0 * u + 0.1 * rng.standard_normal((P, d))
    K = 0.1 * rng.standard_normal((P, d))
    K[0] = 12.0 * u
    ids = np.full(P, 5)
    ids[0] = 0
    comps = adaptive.composites([0], [1], 3, 4)
    k, rec = adaptive.profile(Q, K, ids, comps, 1.0, 8, 0.99)
    assert k == adaptive.C_SPECIAL and rec[1] > 0.99


def test_no_protected_ids_is_h2o_under_ties():
    """Identical keys: every score ties, so the oldest-first and newer-first
    tie rules decide everything; the composite must follow H2O's exactly."""
    rng = np.random.default_rng(8)
    N, P, d = 80, 40, 8
    Q, V = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    K = np.tile(rng.standard_normal(d), (N, 1))
    ids = rng.integers(0, 20, N)
    comp = adaptive.Composite(frozenset(), 6, 9)
    k0, S0, out, ev, kept, S = adaptive.run_composite(comp, Q, K, V, ids, P, 0.5)
    tr = h2o.run_unit(Q, K, V, P, 6, 9, 0.5)
    assert np.array_equal(k0, tr.prefill_kept)
    assert np.array_equal(ev, tr.evicted)


def test_budget_covering_the_prompt_recovers_everything():
    """heavy + recent >= the unprotected prompt: C3 keeps every prompt token,
    and each row's whole softmax (diagonal included) counts: recovery 1."""
    Q, K, V, ids = rand_case(9, 30, 8)
    comps = adaptive.composites([0], [1], 40, 5)
    k, rec = adaptive.profile(Q, K, ids, comps, 0.5, 12, 1.0 - 1e-12)
    assert rec[adaptive.C_FREQUENT] == pytest.approx(1.0, abs=1e-12)
    assert k in (adaptive.C_SPECIAL, adaptive.C_PUNCT, adaptive.C_FREQUENT)


@pytest.mark.parametrize("seed", range(3))
def test_unprotected_part_fills_its_budget_exactly(seed):
    Q, K, V, ids = rand_case(60 + seed, 90, 8, vocab=6)
    heavy, recent, P = 5, 7, 40
    comp = adaptive.Composite(frozenset([0]), heavy, recent)
    k0, S0, out, ev, kept, S = adaptive.run_composite(comp, Q, K, V, ids, P, 0.5)
    free0 = [j for j in k0 if ids[j] != 0]
    assert len(free0) == min(heavy + recent, sum(1 for j in range(P) if ids[j] != 0))
    free = [j for j in kept if ids[j] != 0]
    assert len(free) == min(heavy + recent, sum(1 for j in range(90) if ids[j] != 0))


def test_frequent_composite_has_no_window():
    Q, K, V, ids = rand_case(70, 80, 8, vocab=10)
    comps = adaptive.composites([0], [1], 6, 15)
    c = causal_weights(Q, K, 0.5).sum(axis=0)
    n_prot = sum(1 for j in range(80) if ids[j] in (0, 1))
    assert len(adaptive.prompt_kept(comps[adaptive.C_FREQUENT], c, ids, 80)) == n_prot + 6
    assert len(adaptive.prompt_kept(comps[adaptive.C_LOCAL], c, ids, 80)) == n_prot + 6 + 15


def test_cache_fills_to_its_budget_from_a_short_prompt():
    """A prompt with fewer unprotected tokens than the budget: decode steps
    only add until the unprotected part holds exactly heavy + recent."""
    Q, K, V, ids = rand_case(61, 60, 8, vocab=6)
    heavy, recent, P = 5, 7, 8
    comp = adaptive.Composite(frozenset([0]), heavy, recent)
    k0, S0, out, ev, kept, S = adaptive.run_composite(comp, Q, K, V, ids, P, 0.5)
    assert np.array_equal(k0, np.arange(P))
    free_seen = [j for j in range(60) if ids[j] != 0]
    first_evict = free_seen[heavy + recent]            # the (budget + 1)-th unprotected token
    assert all(e == -1 for e in ev[: first_evict - P])
    assert ev[first_evict - P] != -1
    assert len([j for j in kept if ids[j] != 0]) == heavy + recent


def test_no_protected_ids_is_h2o_with_exact_ties():
    """Keys whose logits are near -1000 get weight exactly 0, so their scores
    tie at 0: the prompt's newer-first and the decode's oldest-first tie rules
    decide; the composite must follow H2O exactly."""
    rng = np.random.default_rng(12)
    N, P, d = 70, 40, 8
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    Q = 5.0 * u + 0.3 * rng.standard_normal((N, d))
    K = rng.standard_normal((N, d))
    dead = rng.choice(N, 50, replace=False)
    K[dead] = -300.0 * u
    V = rng.standard_normal((N, d))
    ids = rng.integers(0, 20, N)
    comp = adaptive.Composite(frozenset(), 18, 5)
    k0, S0, out, ev, kept, S = adaptive.run_composite(comp, Q, K, V, ids, P, 1.0)
    tr = h2o.run_unit(Q, K, V, P, 18, 5, 1.0)
    assert sum(1 for j, s in zip(k0, S0) if j < P - 5 and s == 0) >= 2   # the prompt cut falls among ties
    assert np.array_equal(k0, tr.prefill_kept)
    assert np.array_equal(ev, tr.evicted)
