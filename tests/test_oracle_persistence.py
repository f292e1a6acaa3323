"""Pins of the persistence-count oracle (CPU only).

Closed forms on constructed inputs (identical keys reduce the rule to a
sliding window; one dominant key is kept forever), two trajectories worked by
hand in exact fractions, invariants on random inputs, and a replay of the
recorded per-step weights that rebuilds every history from the definition of
a pivotal step.
"""

import numpy as np
import pytest

from oracle import attention, persistence


def rand_qkv(seed, N, d):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((N, d)) for _ in range(3))


def popcount(x: int) -> int:
    return bin(int(x)).count("1")


@pytest.mark.parametrize("P,T,heavy,recent,window", [(40, 30, 6, 10, 8), (25, 40, 3, 12, 12), (100, 20, 10, 64, 64)])
def test_identical_keys_reduce_to_a_sliding_window(P, T, heavy, recent, window):
    """All logits equal: every weight is exactly 1/|A|, so every token is
    pivotal at every step and every full history has `window` bits; with the
    recent window at least as long as the history window every candidate's
    count is full, the ties go oldest-first, and the cache is always the last
    heavy + recent positions."""
    rng = np.random.default_rng(P + T)
    N, d = P + T, 8
    Q = rng.standard_normal((N, d))
    K = np.tile(rng.standard_normal(d), (N, 1))
    V = rng.standard_normal((N, d))
    B = heavy + recent
    tr = persistence.run_unit(Q, K, V, P, heavy, recent, window, 0.5)
    # prompt histories: key j holds bits 0 .. min(window, P - j) - 1
    for j in range(P):
        assert int(tr.prompt_hist[j]) == (1 << min(window, P - j)) - 1
    assert tr.prefill_kept.tolist() == list(range(P - B, P))
    for s in range(T):
        t = P + s
        assert int(tr.evicted[s]) == (t - B if t - B >= 0 else -1)
    assert sorted(tr.final.pos.tolist()) == list(range(P + T - B, P + T))
    # the last step attends the kept set plus itself, B + 1 tokens, uniformly
    assert np.allclose(tr.out[-1], V[P + T - 1 - B:].mean(axis=0), rtol=0, atol=1e-12)


def test_dominant_key_is_kept_and_the_rest_is_a_window():
    """Key 0 is aligned with every query and far larger than the others: it
    takes almost all the weight at every step (pivotal always), no other token
    reaches 1/|A| (count 0), so the cache is {0} plus the newest tokens."""
    rng = np.random.default_rng(7)
    P, T, d = 30, 25, 16
    heavy, recent, window = 3, 5, 16
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    Q = 4.0 * u + 0.1 * rng.standard_normal((P + T, d))
    K = 0.1 * rng.standard_normal((P + T, d))
    K[0] = 12.0 * u
    V = rng.standard_normal((P + T, d))
    tr = persistence.run_unit(Q, K, V, P, heavy, recent, window, 1.0)
    assert int(tr.prompt_hist[0]) == (1 << window) - 1
    assert all(int(h) == 0 for h in tr.prompt_hist[1:P])
    # heavy part: key 0 plus the newest zero-count candidates
    assert tr.prefill_kept.tolist() == [0] + list(range(P - recent - heavy + 1, P))
    for s in range(T):
        t = P + s
        assert int(tr.evicted[s]) == t - heavy - recent + 1
    assert sorted(tr.final.pos.tolist()) == [0] + list(range(P + T - heavy - recent + 1, P + T))
    assert int(tr.final.hist[0]) == (1 << window) - 1


@pytest.mark.parametrize("seed", range(4))
def test_histories_rebuilt_from_recorded_weights(seed):
    """Each kept token's final history equals the bits recomputed from the
    weights its token received at each of the last `window` steps (prompt rows
    included when the window reaches back into the prompt)."""
    P, T, d = 20, 15, 8
    heavy, recent, window = 4, 5, 24
    Q, K, V = rand_qkv(seed, P + T, d)
    scale = 0.7
    tr = persistence.run_unit(Q, K, V, P, heavy, recent, window, scale, record=True)
    pw = attention.causal_weights(Q[:P], K[:P], scale)
    t_last = P + T - 1
    for pos, h in zip(tr.final.pos, tr.final.hist):
        expect = 0
        for k in range(window):
            step = t_last - k
            if step >= P:
                A, p = tr.steps[step - P]
                w = np.flatnonzero(A == pos)
                if len(w) and p[w[0]] >= 1.0 / len(A):
                    expect |= 1 << k
            elif 0 <= step and pos <= step:
                if pw[step, pos] >= 1.0 / (step + 1):
                    expect |= 1 << k
        assert int(h) == expect, (pos, bin(int(h)), bin(expect))


@pytest.mark.parametrize("seed", range(6))
def test_invariants_on_random_inputs(seed):
    rng = np.random.default_rng(100 + seed)
    P, T, d = int(rng.integers(1, 40)), int(rng.integers(1, 40)), 8
    heavy, recent = int(rng.integers(0, 8)), int(rng.integers(0, 8))
    if heavy + recent == 0:
        heavy = 1
    window = int(rng.integers(1, 65))
    Q, K, V = rand_qkv(seed, P + T, d)
    tr = persistence.run_unit(Q, K, V, P, heavy, recent, window, 0.4, record=True)
    B = heavy + recent
    assert len(tr.prefill_kept) == min(P, B)
    assert set(range(max(0, P - recent), P)) <= set(tr.prefill_kept.tolist())
    for s in range(T):
        t = P + s
        A, p = tr.steps[s]
        assert len(A) == min(P, B) + 1 if s == 0 else True
        if tr.evicted[s] >= 0:
            assert tr.evicted[s] <= t - recent
    assert len(tr.final.pos) == min(P + T, B)
    assert set(range(max(0, P + T - recent), P + T)) <= set(tr.final.pos.tolist())
    assert all(int(h) >> window == 0 for h in tr.final.hist)
    # window = 1: the victim was not pivotal at its last step unless every candidate was
    tr1 = persistence.run_unit(Q, K, V, P, heavy, recent, 1, 0.4, record=True)
    for s in range(T):
        g = int(tr1.evicted[s])
        if g < 0:
            continue
        A, p = tr1.steps[s]
        t = P + s
        piv = p >= 1.0 / len(A)
        cand = A <= t - recent
        if not piv[cand].all():
            assert not piv[np.flatnonzero(A == g)[0]]


def test_victim_order_lowest_count_then_oldest():
    A = np.array([5, 3, 9, 4, 12], dtype=np.int64)
    h = np.array([0b111, 0b1, 0b1, 0b11, 0], dtype=np.uint64)
    # candidates: positions <= 12 - 4 = 8 -> 5, 3, 4; counts 3, 1, 2
    assert persistence.victim(A, h, 12, 4) == 1
    h[3] = 0b10
    # counts 3, 1, 1: equal lowest -> oldest (3)
    assert persistence.victim(A, h, 12, 4) == 1
    h[1] = 0b11
    assert persistence.victim(A, h, 12, 4) == 3


def test_pivotal_band_and_window_checks():
    bits, near = persistence.pivotal(np.array([0.25, 0.25 * (1 + 2e-6), 0.2, 0.3]), 4)
    assert bits.tolist() == [True, True, False, True]
    assert near.tolist() == [True, True, False, False]
    with pytest.raises(ValueError):
        persistence.window_mask(0)
    with pytest.raises(ValueError):
        persistence.window_mask(65)
    assert persistence.window_mask(64) == (1 << 64) - 1


@pytest.mark.parametrize("window", [4, 1])
def test_trajectory_worked_by_hand(window):
    """Two trajectories worked by hand (Scissorhands page, Abstract: pivotal
    tokens are the ones kept; the reading: pivotal = weight at least 1 / |A|,
    count over the last `window` steps, lowest count evicted, oldest first).

    d = 1, scale 1, keys k = (0, 1, 0, 2 | 0, 1), values v_j = j + 1, prompt
    P = 4, one heavy slot and one recent slot.  Query i has e^q = 2 except
    row 3 (e^q = 3), so every weight is a ratio of powers of that base:

      prompt rows   [1], (1, 2)/3, (1, 2, 1)/4, (1, 3, 1, 9)/14
      pivotal       row 0: token 0; row 1: token 1; row 2: token 1; row 3: token 3

    window 4: histories 1000, 0110, 0000, 0001 (bit 3 = row 0); counts
      (1, 2, 0, 1); keep {3} (recent) + {1}.  Step 4 attends {1, 3, 4} with
      (2, 4, 1)/7: token 3 pivotal; histories 1100, 0011, 0000, so 1 and 3
      tie at 2 and the older, 1, leaves; out = (2*2 + 4*4 + 1*5)/7 = 25/7.
      Step 5 attends {3, 4, 5} with (4, 1, 2)/7: 3 pivotal; counts 3, 0 (4
      is the only other candidate) so 4 leaves; out = (16 + 5 + 12)/7 = 33/7.
    window 1: only row 3 counts, so every earlier token has count 0 and the
      newer-first order keeps 2: {2, 3}.  Step 4 attends {2, 3, 4} with
      (1, 4, 1)/6: counts 0, 1 among the candidates 2, 3, so 2 leaves;
      out = (3 + 16 + 5)/6 = 4.  Step 5 as above: 4 leaves, out = 33/7.

    A misread tie order (newest first on equal counts at decode), window
    (counting all steps) or prefill tie order changes a kept set or a victim.
    """
    lnb = np.log([2.0, 2.0, 2.0, 3.0, 2.0, 2.0])
    k = np.array([0.0, 1.0, 0.0, 2.0, 0.0, 1.0])
    Q, K, V = lnb[:, None], k[:, None], (np.arange(6) + 1.0)[:, None]
    tr = persistence.run_unit(Q, K, V, P=4, heavy=1, recent=1, window=window, scale=1.0)
    if window == 4:
        assert [int(h) for h in tr.prompt_hist] == [0b1000, 0b0110, 0b0000, 0b0001]
        assert sorted(tr.prefill_kept.tolist()) == [1, 3]
        assert tr.evicted.tolist() == [1, 4]
        np.testing.assert_allclose(tr.out[:, 0], [25 / 7, 33 / 7], rtol=1e-13)
        final = dict(zip(tr.final.pos.tolist(), (int(h) for h in tr.final.hist)))
        assert final == {3: 0b0111, 5: 0b0000}
    else:
        assert [int(h) for h in tr.prompt_hist] == [0, 0, 0, 1]
        assert sorted(tr.prefill_kept.tolist()) == [2, 3]
        assert tr.evicted.tolist() == [2, 4]
        np.testing.assert_allclose(tr.out[:, 0], [4.0, 33 / 7], rtol=1e-13)
        final = dict(zip(tr.final.pos.tolist(), (int(h) for h in tr.final.hist)))
        assert final == {3: 1, 5: 0}
