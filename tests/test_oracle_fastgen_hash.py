"""Pins of the CPU oracle's FastGen and HashEvict parts (CPU only)."""

import math

import numpy as np
import pytest
import torch

from oracle import fastgen, h2o, hashevict
from tests.test_oracle_h2o import band_mask, causal_mask, rand_qkv, sdpa_rows


def test_full_policy_is_causal_attention():
    P, T, d = 9, 14, 8
    Q, K, V = rand_qkv(5, P + T, d)
    tr = fastgen.run_unit(fastgen.FULL, Q, K, V, P, 0.3, want_prompt_out=True)
    ref = sdpa_rows(Q, K, V, 0.3, causal_mask(P + T))
    np.testing.assert_allclose(tr.out, ref[P:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(tr.prompt_out, ref[:P], rtol=0, atol=1e-12)
    assert (tr.evicted == -1).all()


@pytest.mark.parametrize("P,W", [(20, 6), (4, 9), (12, 12)])
def test_local_policy_is_band_and_equals_h2o_without_heavy(P, W):
    T, d = 25, 8
    Q, K, V = rand_qkv(9 + W, P + T, d, heavy_pos=4)
    tr = fastgen.run_unit(fastgen.LOCAL, Q, K, V, P, 0.3, recent=W)
    ref = sdpa_rows(Q, K, V, 0.3, band_mask(P + T, W + 1))
    np.testing.assert_allclose(tr.out, ref[P:], rtol=0, atol=1e-12)
    hz = h2o.run_unit(Q, K, V, P, heavy=0, recent=W, scale=0.3)
    assert hz.evicted.tolist() == tr.evicted.tolist()
    np.testing.assert_allclose(hz.out, tr.out, rtol=0, atol=1e-12)
    assert sorted(hz.final.pos.tolist()) == tr.final_kept.tolist()


def test_special_policy_is_masked_attention():
    P, T, d = 30, 20, 8
    N = P + T
    Q, K, V = rand_qkv(21, N, d)
    rng = np.random.default_rng(4)
    ids = rng.integers(0, 20, N)
    keep = [0, 1, 2, 3, 7]
    tr = fastgen.run_unit(fastgen.SPECIAL, Q, K, V, P, 0.3, ids=ids, keep_ids=keep)
    is_keep = np.isin(ids, keep)
    mask = causal_mask(N) & (is_keep[None, :] | np.eye(N, dtype=bool))
    ref = sdpa_rows(Q, K, V, 0.3, mask)
    np.testing.assert_allclose(tr.out, ref[P:], rtol=0, atol=1e-12)
    assert tr.prefill_kept.tolist() == [j for j in range(P) if is_keep[j]]
    assert tr.evicted.tolist() == [-1 if is_keep[t] else t for t in range(P, N)]
    assert tr.final_kept.tolist() == [j for j in range(N) if is_keep[j]]


def test_freq_local_keeps_window_and_budget():
    P, T, d, hh, W = 40, 30, 8, 5, 10
    Q, K, V = rand_qkv(33, P + T, d, heavy_pos=7)
    tr = fastgen.run_unit(fastgen.H2O, Q, K, V, P, 0.3, heavy=hh, recent=W)
    assert len(tr.final_kept) == hh + W
    assert set(range(P + T - W, P + T)) <= set(tr.final_kept.tolist())


# ---------------------------------------------------------------- HashEvict

@pytest.mark.parametrize("bits", [16, 32, 64])
def test_sketch_identity_projection_is_sign_bits(bits):
    """W = I (d = bits): bit b of the sketch is [x_b > 0]; bit 0 is the least significant."""
    rng = np.random.default_rng(bits)
    X = rng.standard_normal((50, bits))
    X[3, 5] = 0.0                        # sign(0) -> 0
    X[4, bits - 1] = 1.0                 # the top bit set
    sk = hashevict.sketches(X, np.eye(bits))
    for i in range(50):
        exp = sum(1 << b for b in range(bits) if X[i, b] > 0)
        assert int(sk[i]) == exp
    assert int(sk[4]) >> (bits - 1) == 1


def test_sketch_sign_is_exact_for_cancelling_sums():
    """A plain float64 dot loses the +1 here; the exact sign is positive."""
    x = np.array([[2.0 ** 60, 1.0, -(2.0 ** 60)], [2.0 ** 60, -1.0, -(2.0 ** 60)]])
    W = np.ones((3, 1))
    assert (x[0, 0] + x[0, 1]) + x[0, 2] == 0.0           # left-to-right float64 loses the +1
    sk = hashevict.sketches(x, W)
    assert int(sk[0]) == 1 and int(sk[1]) == 0


def test_hamming_matches_bit_counting():
    rng = np.random.default_rng(1)
    a = rng.integers(0, 2 ** 32, 200, dtype=np.uint64)
    b = rng.integers(0, 2 ** 32, 200, dtype=np.uint64)
    h = hashevict.hamming(a, b)
    assert h.tolist() == [bin(int(x) ^ int(y)).count("1") for x, y in zip(a, b)]


def test_sketch_distance_tracks_angle():
    """Sign random projections: P[bit differs] = angle / pi (the SimHash property),
    so the mean distance over 32 Gaussian columns is 32 angle / pi."""
    rng = np.random.default_rng(2)
    d, n = 128, 4000
    for theta in (0.3, 1.0, 2.0):
        W = rng.standard_normal((d, 32))
        X = rng.standard_normal((n, d))
        X /= np.linalg.norm(X, axis=1, keepdims=True)
        Z = rng.standard_normal((n, d))
        Z -= (Z * X).sum(1, keepdims=True) * X
        Z /= np.linalg.norm(Z, axis=1, keepdims=True)
        Y = math.cos(theta) * X + math.sin(theta) * Z
        h = hashevict.hamming(hashevict.sketches(X, W), hashevict.sketches(Y, W))
        assert abs(h.mean() - 32 * theta / math.pi) < 0.35


def test_identical_sketches_give_fifo_band():
    """All keys identical: every distance ties, the oldest goes, so the cache is
    a window of the last B positions."""
    P, T, d, B = 20, 30, 8, 7
    N = P + T
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((N, d))
    K = np.tile(rng.standard_normal(d), (N, 1))
    V = rng.standard_normal((N, d))
    W = rng.standard_normal((d, 32))
    tr = hashevict.run_unit(Q, K, V, W, P, B, 0.3)
    assert tr.prefill_kept.tolist() == list(range(P - B, P))
    assert tr.evicted.tolist() == [t - B for t in range(P, N)]
    ref = sdpa_rows(Q, K, V, 0.3, band_mask(N, B))
    np.testing.assert_allclose(tr.out, ref[P:], rtol=0, atol=1e-12)


def test_farthest_brute_force():
    rng = np.random.default_rng(6)
    ksk = rng.integers(0, 16, 40, dtype=np.uint64)     # small values -> many ties
    for _ in range(50):
        cache = rng.choice(40, 12, replace=False)
        q = int(rng.integers(0, 16))
        v = hashevict.farthest(q, cache, ksk)
        dist = [bin(q ^ int(ksk[p])).count("1") for p in cache]
        best = max(dist)
        assert dist[v] == best
        assert cache[v] == min(p for p, h in zip(cache, dist) if h == best)


def test_hash_budget_above_context_is_full_attention():
    P, T, d = 10, 12, 8
    Q, K, V = rand_qkv(8, P + T, d)
    W = np.random.default_rng(9).standard_normal((d, 32))
    tr = hashevict.run_unit(Q, K, V, W, P, P + T, 0.3)
    ref = sdpa_rows(Q, K, V, 0.3, causal_mask(P + T))
    np.testing.assert_allclose(tr.out, ref[P:], rtol=0, atol=1e-12)
    assert (tr.evicted == -1).all()


def test_hash_cache_invariants():
    P, T, d, B = 40, 40, 16, 12
    Q, K, V = rand_qkv(10, P + T, d)
    W = np.random.default_rng(11).standard_normal((d, 32))
    tr = hashevict.run_unit(Q, K, V, W, P, B, 0.25)
    assert len(tr.prefill_kept) == B and len(set(tr.prefill_kept.tolist())) == B
    assert len(tr.final_kept) == B and (P + T - 1) in tr.final_kept.tolist()
    # every evicted position was in the cache and never comes back
    seen = set(tr.prefill_kept.tolist())
    for s, e in enumerate(tr.evicted):
        assert e in seen
        seen.discard(int(e)); seen.add(P + s)
    assert seen == set(tr.final_kept.tolist())


@pytest.mark.parametrize("policy", [fastgen.FULL, fastgen.LOCAL, fastgen.SPECIAL, fastgen.H2O, "hash"])
def test_zero_decode_steps_is_the_prefill_alone(policy):
    """steps=0 runs the prefill only: empty outputs and logs, the same prompt
    cache as the full run."""
    P, T, d = 24, 9, 8
    Q, K, V = rand_qkv(31, P + T, d, heavy_pos=3)
    ids = np.random.default_rng(2).integers(0, 20, P + T)
    if policy == "hash":
        W = np.random.default_rng(3).standard_normal((d, 32))
        zero = hashevict.run_unit(Q, K, V, W, P, 10, 0.3, steps=0)
        full = hashevict.run_unit(Q, K, V, W, P, 10, 0.3)
    else:
        kw = dict(heavy=4, recent=6, ids=ids, keep_ids=[0, 1, 5])
        zero = fastgen.run_unit(policy, Q, K, V, P, 0.3, steps=0, **kw)
        full = fastgen.run_unit(policy, Q, K, V, P, 0.3, **kw)
    assert zero.out.shape == (0, d) and len(zero.evicted) == 0
    assert zero.prefill_kept.tolist() == full.prefill_kept.tolist()
