"""Pins for the 4-bit cache format oracle and its use by the H2O and
persistence oracles ([SH] Abstract: eviction combined with 4-bit quantisation).

Each pin checks the oracle against something other than its own code: exact
integer grids, the half-to-even rule, a brute-force nearest-grid-point search,
the rounding error bound of a uniform grid, and trajectories whose cached rows
the format holds exactly.
"""

import numpy as np
import pytest

from oracle import h2o, persistence, quant
from oracle.attention import attend


def test_integer_grid_is_exact():
    # amax 7 -> scale = 7 * fl32(1/7), which rounds to exactly 1.0 in float32;
    # every integer in [-7, 7] is then its own code and reads back exactly.
    row = np.tile(np.arange(-7, 8, dtype=np.float64), 5)[:64].reshape(1, 64)
    row[0, 31] = 7.0
    row[0, 63] = -7.0
    codes, scale = quant.quantize_rows(row)
    assert scale.dtype == np.float32 and np.all(scale == 1.0)
    assert np.array_equal(codes.astype(np.float64), row)
    assert np.array_equal(quant.roundtrip(row), row)


def test_half_to_even():
    g = np.zeros((1, 32))
    g[0, 0] = 7.0
    g[0, 1:9] = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 6.5]
    codes, scale = quant.quantize_rows(g)
    assert scale[0, 0] == 1.0
    assert codes[0, 1:9].tolist() == [0, 2, 2, 4, 0, -2, -2, 6]


def test_zero_group_and_sign():
    x = np.zeros((2, 64))
    x[0, 32:] = -np.linspace(0.1, 3.0, 32)
    codes, scale = quant.quantize_rows(x)
    assert scale[0, 0] == 0 and scale[1, 0] == 0 and scale[1, 1] == 0
    assert not codes[0, :32].any() and not codes[1].any()
    assert np.all(codes[0, 32:] <= 0) and codes[0, 63] == -7
    assert np.array_equal(quant.roundtrip(x)[1], np.zeros(64))


def test_groups_are_independent():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 128))
    x[:, 32:64] *= 1000.0
    x[:, 96:] *= 1e-3
    codes, scale = quant.quantize_rows(x)
    for gi in range(4):
        sl = slice(32 * gi, 32 * gi + 32)
        c2, s2 = quant.quantize_rows(x[:, sl])
        assert np.array_equal(codes[:, sl], c2) and np.array_equal(scale[:, gi], s2[:, 0])
        amax = np.max(np.abs(x[:, sl].astype(np.float32)), axis=1)
        np.testing.assert_allclose(scale[:, gi], amax / 7.0, rtol=2e-7)
        # the largest element of each group takes the extreme code
        assert np.all(np.max(np.abs(codes[:, sl]), axis=1) == 7)


def test_nearest_grid_point_by_brute_force():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 64)).astype(np.float32).astype(np.float64)
    codes, scale = quant.quantize_rows(x)
    grid = np.arange(-7, 8, dtype=np.float64)
    for r in range(x.shape[0]):
        for e in range(x.shape[1]):
            s = float(scale[r, e // 32])
            q = x[r, e] / s
            if abs(abs(q - np.floor(q)) - 0.5) < 1e-5:
                continue            # a tie up to float32 rounding: either side is right
            best = grid[np.argmin(np.abs(x[r, e] - grid * s))]
            assert codes[r, e] == best, (r, e)


def test_error_bound_and_idempotence():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((256, 128)) * rng.uniform(0.01, 50, (256, 1))).astype(np.float32)
    codes, scale = quant.quantize_rows(x)
    y = quant.dequantize_rows(codes, scale)
    s = np.repeat(scale.astype(np.float64), 32, axis=1)
    # rounding to a grid of step s: half a step, plus the float32 quotient's error
    assert np.all(np.abs(y - x) <= 0.5 * s + np.abs(x) * 2.0 ** -21)
    codes2, _ = quant.quantize_rows(y)
    assert np.array_equal(codes, codes2)
    with pytest.raises(ValueError):
        quant.quantize_rows(np.ones((1, 48)))


def _grid_rows(rng, n, d):
    """Rows the format holds exactly: integers in [-7, 7] with a 7 in every group."""
    X = rng.integers(-7, 8, size=(n, d)).astype(np.float64)
    X[:, ::32] = 7.0
    return X


def test_h2o_trajectory_unchanged_when_the_format_is_exact():
    rng = np.random.default_rng(5)
    N, P, d = 40, 24, 64
    Q = rng.standard_normal((N, d)) * 0.05
    K, V = _grid_rows(rng, N, d), _grid_rows(rng, N, d)
    a = h2o.run_unit(Q, K, V, P, 6, 4, d ** -0.5)
    b = h2o.run_unit(Q, K, V, P, 6, 4, d ** -0.5, Kc=quant.roundtrip(K), Vc=quant.roundtrip(V))
    assert np.array_equal(a.evicted, b.evicted)
    assert np.array_equal(a.out, b.out)


def test_step_token_is_read_at_full_precision():
    # Cached slots read Kc / Vc; the step's own token reads K / V.  Poisoning the
    # slot copy of the last position must leave every output finite, and the
    # first step's output must be the attention over (cached copies, own row).
    rng = np.random.default_rng(9)
    N, P, d = 30, 20, 64
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    Kc, Vc = quant.roundtrip(K), quant.roundtrip(V)
    Kc[N - 1] = np.nan
    Vc[N - 1] = np.nan
    tr = h2o.run_unit(Q, K, V, P, 5, 5, d ** -0.5, Kc=Kc, Vc=Vc)
    assert np.all(np.isfinite(tr.out))
    kept = tr.prefill_kept
    Ks = np.vstack([quant.roundtrip(K)[kept], K[P]])
    Vs = np.vstack([quant.roundtrip(V)[kept], V[P]])
    np.testing.assert_allclose(tr.out[0], attend(Q[P], Ks, Vs, d ** -0.5)[1], rtol=0, atol=1e-12)
    tp = persistence.run_unit(Q, K, V, P, 5, 5, 8, d ** -0.5, Kc=Kc, Vc=Vc)
    assert np.all(np.isfinite(tp.out))
    kept = tp.prefill_kept
    Ks = np.vstack([quant.roundtrip(K)[kept], K[P]])
    Vs = np.vstack([quant.roundtrip(V)[kept], V[P]])
    np.testing.assert_allclose(tp.out[0], attend(Q[P], Ks, Vs, d ** -0.5)[1], rtol=0, atol=1e-12)
    # and the lossy copy does change what the cache attends to
    assert np.abs(tr.out - h2o.run_unit(Q, K, V, P, 5, 5, d ** -0.5).out).max() > 1e-4


def test_hashevict_reads_every_attended_row_from_its_slot():
    """HashEvict attends the cache after inserting token t: with 4-bit slots
    every attended row, t included, is the slot copy; the sketches (from the
    inputs) and hence every eviction are those of the full-precision run."""
    from oracle import hashevict
    rng = np.random.default_rng(13)
    N, P, d, B = 50, 30, 64, 12
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    W = rng.standard_normal((d, 32))
    Kc, Vc = quant.roundtrip(K), quant.roundtrip(V)
    full = hashevict.run_unit(Q, K, V, W, P, B, d ** -0.5)
    q4 = hashevict.run_unit(Q, K, V, W, P, B, d ** -0.5, Kc=Kc, Vc=Vc)
    assert np.array_equal(full.evicted, q4.evicted) and np.array_equal(full.final_kept, q4.final_kept)
    # first decode step: the cache after the replacement holds P in some slot
    cache = list(hashevict.replay_prompt(q4.qsk, q4.ksk, P, B))
    v = hashevict.farthest(int(q4.qsk[P]), np.array(cache, dtype=np.int64), q4.ksk)
    cache[v] = P
    A = np.array(cache, dtype=np.int64)
    np.testing.assert_allclose(q4.out[0], attend(Q[P], Kc[A], Vc[A], d ** -0.5)[1], rtol=0, atol=1e-12)
    assert np.abs(q4.out - full.out).max() > 1e-4
    # rows the format holds exactly change nothing
    Kg, Vg = _grid_rows(rng, N, d), _grid_rows(rng, N, d)
    a = hashevict.run_unit(Q, Kg, Vg, W, P, B, d ** -0.5)
    b = hashevict.run_unit(Q, Kg, Vg, W, P, B, d ** -0.5, Kc=quant.roundtrip(Kg), Vc=quant.roundtrip(Vg))
    assert np.array_equal(a.out, b.out)
