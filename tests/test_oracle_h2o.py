"""Pins of the CPU oracle's attention and H2O parts (CPU only).

Each test ties the oracle to something other than itself: a textbook routine
(torch's scaled_dot_product_attention in float64), a closed form, an invariant
or brute-force enumeration.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention, h2o


def sdpa_rows(Q, K, V, scale, mask):
    """Textbook attention (torch, float64) with a boolean mask [N, N] (True = attend)."""
    q = torch.from_numpy(Q)[None, None]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    m = torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


def causal_mask(N):
    return np.tril(np.ones((N, N), dtype=bool))


def band_mask(N, width):
    """Row t sees positions [t - width + 1, t]."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    return (j <= i) & (j > i - width)


def rand_qkv(seed, N, d, heavy_pos=0):
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    if heavy_pos:
        u = rng.standard_normal(d)
        u *= np.sqrt(d) / np.linalg.norm(u)
        idx = rng.choice(N, heavy_pos, replace=False)
        K[idx] += 3 * u
    return Q, K, V


def test_causal_attention_matches_sdpa():
    Q, K, V = rand_qkv(1, 37, 16)
    scale = 1 / np.sqrt(16)
    _, out = attention.causal_attention(Q, K, V, scale)
    np.testing.assert_allclose(out, sdpa_rows(Q, K, V, scale, causal_mask(37)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("P,T,d", [(12, 20, 8), (1, 9, 4), (30, 1, 16)])
def test_budget_at_least_context_is_full_attention(P, T, d):
    """Budget >= context: every decode output is the causal attention row."""
    Q, K, V = rand_qkv(P * 100 + T, P + T, d, heavy_pos=3)
    scale = 1 / np.sqrt(d)
    N = P + T
    tr = h2o.run_unit(Q, K, V, P, heavy=N, recent=0, scale=scale, want_prompt_out=True)
    ref = sdpa_rows(Q, K, V, scale, causal_mask(N))
    np.testing.assert_allclose(tr.out, ref[P:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(tr.prompt_out, ref[:P], rtol=0, atol=1e-12)
    assert (tr.evicted == -1).all()
    assert sorted(tr.final.pos.tolist()) == list(range(N))
    # the same with the budget split between heavy and recent parts
    tr2 = h2o.run_unit(Q, K, V, P, heavy=N // 2, recent=N - N // 2, scale=scale)
    np.testing.assert_allclose(tr2.out, ref[P:], rtol=0, atol=1e-12)


@pytest.mark.parametrize("P,T,r", [(20, 30, 5), (6, 20, 6), (3, 15, 4), (16, 16, 1)])
def test_no_heavy_slots_is_sliding_window(P, T, r):
    """heavy = 0: step t attends over [t - r, t] (a band of width r + 1)."""
    N, d = P + T, 8
    Q, K, V = rand_qkv(7 + P, N, d, heavy_pos=4)
    scale = 1 / np.sqrt(d)
    tr = h2o.run_unit(Q, K, V, P, heavy=0, recent=r, scale=scale)
    ref = sdpa_rows(Q, K, V, scale, band_mask(N, r + 1))
    np.testing.assert_allclose(tr.out, ref[P:], rtol=0, atol=1e-12)
    exp_ev = [t - r if t - r >= 0 and t >= r else -1 for t in range(P, N)]
    # the cache only overflows once it holds r tokens
    assert tr.evicted.tolist() == exp_ev


def harmonic(n):
    return sum(Fraction(1, k) for k in range(1, n + 1))


def test_identical_keys_column_scores_closed_form():
    """Identical keys: every row's weights are uniform, so c_j = H_P - H_j."""
    P, d = 25, 8
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((P, d))
    K = np.tile(rng.standard_normal(d), (P, 1))
    c = h2o.prefill_column_scores(Q, K, 0.3)
    HP = harmonic(P)
    exp = np.array([float(HP - harmonic(j)) for j in range(P)])
    np.testing.assert_allclose(c, exp, rtol=1e-13)
    # strictly decreasing, so the heavy part is the oldest positions
    kept = h2o.prefill_select(c, heavy=4, recent=5)
    assert kept.tolist() == [0, 1, 2, 3] + list(range(20, 25))


@pytest.mark.parametrize("P,T,hh,r", [(30, 40, 4, 6), (12, 30, 2, 1), (40, 10, 7, 0)])
def test_identical_keys_full_trajectory(P, T, hh, r):
    """Identical keys: all weights uniform.  Closed form of the whole run:
    the heavy set stays [0, hh), the token leaving the recent window is the
    victim (t - r at step t), and each output is the mean of V over
    [0, hh) plus [t - r, t]."""
    N, d = P + T, 6
    rng = np.random.default_rng(11)
    Q = rng.standard_normal((N, d))
    K = np.tile(rng.standard_normal(d), (N, 1))
    V = rng.standard_normal((N, d))
    tr = h2o.run_unit(Q, K, V, P, heavy=hh, recent=r, scale=0.5)
    for s in range(T):
        t = P + s
        A = list(range(hh)) + list(range(t - r, t + 1))
        np.testing.assert_allclose(tr.out[s], V[A].mean(axis=0), rtol=0, atol=1e-12)
        assert tr.evicted[s] == t - r
    assert sorted(tr.final.pos.tolist()) == list(range(hh)) + list(range(N - r, N))


def test_ties_evict_oldest_and_prefill_keeps_newer():
    A = np.array([3, 9, 1, 7, 12])
    S = np.array([0.5, 0.25, 0.25, 0.25, 0.1])
    # t = 12, recent = 1: candidates are positions <= 11 -> 3, 9, 1, 7; lowest 0.25 at 9, 1, 7
    assert A[h2o.h2o_victim(A, S, t=12, recent=1)] == 1
    c = np.array([0.5, 0.7, 0.5, 0.5, 0.9, 0.1, 0.2])
    # candidates [0, 5); heavy 3: 0.9 (4), 0.7 (1), then one of the 0.5s -> the newest (3)
    assert h2o.prefill_select(c, heavy=3, recent=2).tolist() == [1, 3, 4, 5, 6]


def check_invariants(Q, K, V, P, hh, r, scale):
    """Run step by step and check the cache invariants after prefill and every step."""
    B = hh + r
    cache, c = h2o.prefill(Q[:P], K[:P], hh, r, scale)
    dropped = sum(c[j] for j in range(P) if j not in set(cache.pos.tolist()))
    evicted_mass = 0.0
    rows = P

    def inv(t):
        pos = cache.pos.tolist()
        assert len(pos) <= B
        assert len(set(pos)) == len(pos)
        assert all(0 <= p <= t for p in pos)
        assert set(range(max(0, t - r + 1), t + 1)) <= set(pos)
        assert (cache.S > 0).all()
        total = cache.S.sum() + dropped + evicted_mass
        assert abs(total - rows) <= 1e-10 * rows

    inv(P - 1)
    for t in range(P, Q.shape[0]):
        _, A, S_A = h2o.attend_step(cache, t, Q[t], K, V, scale)
        rows += 1
        if len(A) > B:
            i = h2o.h2o_victim(A, S_A, t, r)
            evicted_mass += S_A[i]
            cache = h2o.remove(A, S_A, i)
        else:
            cache = h2o.Cache(A, S_A)
        inv(t)


@pytest.mark.parametrize("seed,P,T,hh,r", [(0, 40, 60, 5, 5), (1, 8, 50, 3, 4), (2, 64, 64, 16, 16),
                                           (3, 20, 30, 7, 0), (4, 5, 30, 0, 3)])
def test_cache_invariants_and_score_conservation(seed, P, T, hh, r):
    Q, K, V = rand_qkv(seed, P + T, 16, heavy_pos=(P + T) // 10)
    check_invariants(Q, K, V, P, hh, r, 0.25)


def test_prefill_selection_maximises_retained_score_brute_force():
    """Over every admissible kept set (recent window kept, heavy-many others), the
    oracle's set retains the most score mass; it is the unique maximiser."""
    for seed in range(6):
        P, d, hh, r = 11, 4, 3, 2
        Q, K, _ = rand_qkv(100 + seed, P, d, heavy_pos=2)
        c = h2o.prefill_column_scores(Q, K, 0.5)
        kept = set(h2o.prefill_select(c, hh, r).tolist())
        best, best_sets = -1.0, []
        for sub in itertools.combinations(range(P - r), hh):
            m = sum(c[j] for j in sub)
            if m > best + 1e-15:
                best, best_sets = m, [set(sub)]
            elif abs(m - best) <= 1e-15:
                best_sets.append(set(sub))
        assert len(best_sets) == 1
        assert kept == best_sets[0] | set(range(P - r, P))


def test_decode_eviction_maximises_retained_score_brute_force():
    """At every decode step, evicting the oracle's victim retains the most score
    mass over all admissible single victims (outside the recent window)."""
    P, T, d, hh, r = 10, 6, 4, 3, 2
    for seed in range(5):
        Q, K, V = rand_qkv(200 + seed, P + T, d, heavy_pos=3)
        cache, _ = h2o.prefill(Q[:P], K[:P], hh, r, 0.5)
        for t in range(P, P + T):
            _, A, S_A = h2o.attend_step(cache, t, Q[t], K, V, 0.5)
            admissible = [i for i in range(len(A)) if A[i] <= t - r]
            retained = {i: S_A.sum() - S_A[i] for i in admissible}
            best = max(retained.values())
            i = h2o.h2o_victim(A, S_A, t, r)
            assert retained[i] == best
            winners = [j for j in admissible if retained[j] == best]
            assert A[i] == min(A[j] for j in winners)
            cache = h2o.remove(A, S_A, i)


def test_worked_example_with_distinct_keys():
    """A trajectory worked by hand on distinct keys (H2O review page,
    proposed method: accumulated attention decides which tokens stay).

    d = 1, scale 1, keys k = (0, 1, 2 | 1, 0), queries e^q = (2, 2, 2 | 27, 2),
    values v = (1, 2, 3 | 4, 5); prompt P = 3, one heavy and one recent slot.
    Every weight is a ratio of powers of the query's base, so each number
    below is an exact fraction:

      prompt rows   [1], [1, 2]/3, [1, 2, 4]/7
      column sums   c = (31/21, 20/21, 4/7); keep {2} (recent) + {0} (top c)
      step 3        attends {0, 2, 3}: e = (1, 729, 27)/757, o = 2296/757;
                    S0 = 31/21 + 1/757 < S2 = 4/7 + 729/757, so 0 goes
                    (without this step's weights 2 would go: the step adds
                    its weights before it evicts), token 3 keeps 27/757
      step 4        attends {2, 3, 4}: e = (4, 2, 1)/7, o = 25/7;
                    S3 = 27/757 + 2/7 < S2, so 3 goes; S4 = 1/7
      final         {2, 4} with S = (4/7 + 729/757 + 4/7, 1/7)
    """
    ln = np.log
    K = np.array([[0.0], [1.0], [2.0], [1.0], [0.0]])
    Q = np.array([[ln(2.0)], [ln(2.0)], [ln(2.0)], [ln(27.0)], [ln(2.0)]])
    V = np.array([[1.0], [2.0], [3.0], [4.0], [5.0]])
    tr = h2o.run_unit(Q, K, V, 3, 1, 1, 1.0)
    F = Fraction
    close = lambda a, b: np.allclose(np.asarray(a, dtype=float), [float(x) for x in b], rtol=1e-13, atol=0)
    assert close(tr.column_scores, [F(31, 21), F(20, 21), F(4, 7)])
    assert list(tr.prefill_kept) == [0, 2]
    assert close(tr.prefill_scores, [F(31, 21), F(4, 7)])
    assert close(tr.out[:, 0], [F(2296, 757), F(25, 7)])
    assert list(tr.evicted) == [0, 3]
    assert close(tr.evicted_score, [F(31, 21) + F(1, 757), F(27, 757) + F(2, 7)])
    assert list(tr.final.pos) == [2, 4]
    assert close(tr.final.S, [F(4, 7) + F(729, 757) + F(4, 7), F(1, 7)])
