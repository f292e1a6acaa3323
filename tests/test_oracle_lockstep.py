"""Self-tests of the lockstep checker: it must accept the oracle's own run, accept an
in-band near-tie (and count it), and reject a wrong victim, a perturbed score and a
perturbed output (CPU only)."""

import numpy as np

from oracle import h2o, hashevict, lockstep
from tests.test_oracle_h2o import rand_qkv

P, T, D, HH, R, SC = 40, 30, 16, 6, 6, 0.25


def oracle_as_gpu():
    Q, K, V = rand_qkv(77, P + T, D, heavy_pos=7)
    tr = h2o.run_unit(Q, K, V, P, HH, R, SC)
    g = lockstep.GpuUnit(prefill_pos=tr.prefill_kept.copy(), evicted=tr.evicted.copy(),
                         out=tr.out.copy(), final_pos=tr.final.pos.copy(),
                         prefill_S=tr.prefill_scores.copy(), final_S=tr.final.S.copy())
    return (Q, K, V), tr, g


def test_oracle_log_passes():
    (Q, K, V), tr, g = oracle_as_gpu()
    rep = lockstep.check_h2o(Q, K, V, P, HH, R, SC, g)
    assert rep.ok, rep.failures
    assert rep.adopted == 0 and rep.decisions == T


def test_wrong_victim_fails():
    (Q, K, V), tr, g = oracle_as_gpu()
    s = 5
    t = P + s
    _, A, S_A = None, None, None
    # replay to step s to find a candidate that is clearly not minimal
    cache = h2o.Cache(tr.prefill_kept.copy(), tr.prefill_scores.copy())
    for k in range(s + 1):
        _, A, S_A = h2o.attend_step(cache, P + k, Q[P + k], K, V, SC)
        i = h2o.h2o_victim(A, S_A, P + k, R)
        if k < s:
            cache = h2o.remove(A, S_A, i)
    cand = h2o.h2o_candidates(A, t, R)
    worst = cand[np.argmax(S_A[cand])]
    assert S_A[worst] > S_A[i] * (1 + 1e-3)
    g.evicted[s] = A[worst]
    rep = lockstep.check_h2o(Q, K, V, P, HH, R, SC, g)
    assert not rep.ok
    assert any(f.startswith(f"step {s}:") for f in rep.failures)


def test_perturbed_score_fails():
    (Q, K, V), tr, g = oracle_as_gpu()
    g.final_S[3] *= 1 + 2e-5
    assert not lockstep.check_h2o(Q, K, V, P, HH, R, SC, g).ok
    (Q, K, V), tr, g = oracle_as_gpu()
    g.prefill_S[0] *= 1 - 2e-5
    assert not lockstep.check_h2o(Q, K, V, P, HH, R, SC, g).ok


def test_perturbed_output_fails():
    (Q, K, V), tr, g = oracle_as_gpu()
    g.out[7, 2] += 3e-3 * np.max(np.abs(tr.out[7]))
    rep = lockstep.check_h2o(Q, K, V, P, HH, R, SC, g)
    assert not rep.ok and any("output" in f for f in rep.failures)
    (Q, K, V), tr, g = oracle_as_gpu()
    g.out[7, 2] += 1e-3 * np.max(np.abs(tr.out[7]))
    assert lockstep.check_h2o(Q, K, V, P, HH, R, SC, g).ok


def test_near_tie_victim_is_accepted_far_one_is_not():
    A = np.array([2, 5, 8, 11])
    S = np.array([0.30, 0.30000001, 0.2, 0.9])
    cand = np.array([0, 1, 2])           # position 11 is in the recent window
    i_ref = 2
    assert not lockstep.accept_h2o_victim(A, S, cand, i_ref, 5)
    S2 = np.array([0.30, 0.2 * (1 + 5e-7), 0.2, 0.9])
    assert lockstep.accept_h2o_victim(A, S2, cand, i_ref, 5)
    assert not lockstep.accept_h2o_victim(A, S2, cand, i_ref, 11)   # recent: never admissible
    assert not lockstep.accept_h2o_victim(A, S2, cand, i_ref, 99)   # not in the cache


def test_prefill_near_tie_set_is_adopted():
    c = np.array([0.9, 0.5, 0.5 * (1 + 3e-7), 0.1, 0.2, 0.3, 0.4])
    # candidates [0, 5); heavy 2 -> oracle keeps 0 and 2; GPU keeps 0 and 1 (in band)
    rep = lockstep.UnitReport()
    kept = lockstep.check_prefill_set(rep, c, np.array([0, 1, 5, 6]), heavy=2, recent=2)
    assert rep.ok and rep.adopted == 1 and kept.tolist() == [0, 1, 5, 6]
    rep = lockstep.UnitReport()
    lockstep.check_prefill_set(rep, c, np.array([0, 4, 5, 6]), heavy=2, recent=2)
    assert not rep.ok


def test_hash_checker_accepts_oracle_and_rejects_wrong_victim():
    Pq, Tq, B = 30, 20, 10
    Q, K, V = rand_qkv(5, Pq + Tq, 16)
    W = np.random.default_rng(3).standard_normal((16, 32))
    tr = hashevict.run_unit(Q, K, V, W, Pq, B, 0.25)
    g = lockstep.GpuUnit(prefill_pos=tr.prefill_kept, evicted=tr.evicted.copy(), out=tr.out,
                         final_pos=tr.final_kept)
    assert lockstep.check_hash(Q, K, V, W, Pq, B, 0.25, g).ok
    # pick a cached position at a strictly smaller distance than the maximum at step 0
    cache = hashevict.replay_prompt(tr.qsk, tr.ksk, Pq, B)
    h = hashevict.hamming(np.uint64(tr.qsk[Pq]), tr.ksk[cache])
    near = cache[np.argmin(h)]
    assert h.min() < h.max()
    g.evicted[0] = near
    assert not lockstep.check_hash(Q, K, V, W, Pq, B, 0.25, g).ok


def persist_gpu_unit(tr, P):
    """A GPU log made from the persistence oracle's own trajectory (histories
    exported as the raw bits of float64 scores, as the library does)."""
    return lockstep.GpuUnit(prefill_pos=tr.prefill_kept.copy(), evicted=tr.evicted.copy(), out=tr.out.copy(),
                            final_pos=tr.final.pos.copy(),
                            prefill_S=tr.prefill_hist.astype(np.uint64).view(np.float64).copy(),
                            final_S=tr.final.hist.astype(np.uint64).view(np.float64).copy())


def test_persist_checker_accepts_oracle_and_rejects_mistakes():
    from oracle import persistence
    rng = np.random.default_rng(11)
    P, T, d, hh, r, w = 40, 30, 8, 6, 6, 16
    Q, K, V = (rng.standard_normal((P + T, d)) for _ in range(3))
    tr = persistence.run_unit(Q, K, V, P, hh, r, w, 0.6)
    g = persist_gpu_unit(tr, P)
    rep = lockstep.check_persist(Q, K, V, P, hh, r, w, 0.6, g)
    assert rep.ok and rep.adopted == 0 and rep.decisions == T, rep.failures
    # a different victim at one step (a token that stays kept in the oracle)
    s = int(np.flatnonzero(tr.evicted >= 0)[3])
    bad = persistence_victim_alternative(Q, K, V, P, hh, r, w, tr, s)
    g2 = persist_gpu_unit(tr, P)
    g2.evicted[s] = bad
    assert not lockstep.check_persist(Q, K, V, P, hh, r, w, 0.6, g2).ok
    # one flipped history bit in the final export
    g3 = persist_gpu_unit(tr, P)
    bits = g3.final_S.view(np.uint64)
    bits[0] ^= np.uint64(1)
    assert not lockstep.check_persist(Q, K, V, P, hh, r, w, 0.6, g3).ok
    # one flipped bit in the prompt export
    g4 = persist_gpu_unit(tr, P)
    g4.prefill_S.view(np.uint64)[2] ^= np.uint64(4)
    assert not lockstep.check_persist(Q, K, V, P, hh, r, w, 0.6, g4).ok
    # a prompt kept set with one heavy token swapped for a dropped one
    g5 = persist_gpu_unit(tr, P)
    heavy_kept = [j for j in tr.prefill_kept if j < P - r]
    dropped = sorted(set(range(P - r)) - set(tr.prefill_kept.tolist()))
    cnt = persistence.count(tr.prompt_hist)
    lowest_dropped = min(dropped, key=lambda j: (cnt[j], j))
    strongest_kept = max(heavy_kept, key=lambda j: (cnt[j], j))
    if cnt[lowest_dropped] < cnt[strongest_kept]:
        g5.prefill_pos[list(g5.prefill_pos).index(strongest_kept)] = lowest_dropped
        assert not lockstep.check_persist(Q, K, V, P, hh, r, w, 0.6, g5).ok


def persistence_victim_alternative(Q, K, V, P, hh, r, w, tr, s):
    """A candidate at step s other than the oracle's victim, with a higher count."""
    from oracle import persistence
    cache, _, _ = persistence.prefill(Q[:P], K[:P], hh, r, w, 0.6)
    for k in range(s + 1):
        t = P + k
        _, A, h, a, _ = persistence.attend_step(cache, t, Q[t], K, V, 0.6, w)
        i = persistence.victim(A, h, t, r)
        if k == s:
            cand = persistence.candidates(A, t, r)
            c = persistence.count(h)
            others = [j for j in cand if j != i and c[j] > c[i]]
            return int(A[others[0]])
        cache = persistence.remove(A, h, a, i)


def test_persist_checker_accepts_ambiguous_choice():
    """Identical keys: every weight sits exactly on the threshold, so every bit
    is ambiguous; any candidate is then an admissible victim and is adopted."""
    from oracle import persistence
    rng = np.random.default_rng(3)
    P, T, d, hh, r, w = 30, 10, 8, 4, 8, 8
    Q = rng.standard_normal((P + T, d))
    K = np.tile(rng.standard_normal(d), (P + T, 1))
    V = rng.standard_normal((P + T, d))
    tr = persistence.run_unit(Q, K, V, P, hh, r, w, 0.5)
    g = persist_gpu_unit(tr, P)
    # at step 0 evict the newest candidate instead of the oldest
    t = P
    g.evicted[0] = t - r
    rep = lockstep.check_persist(Q, K, V, P, hh, r, w, 0.5, g, steps=1)
    assert rep.adopted == 1
    assert not any("GPU evicted" in f for f in rep.failures), rep.failures


def adaptive_case(seed=2, P=40, T=30, d=8):
    from oracle import adaptive
    rng = np.random.default_rng(seed)
    N = P + T
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    ids = rng.integers(0, 8, N)
    return Q, K, V, ids


def adaptive_gpu_unit(tr):
    import numpy as np
    fin = np.array(tr.final_kept)
    S = np.where(tr.protected_final, np.inf, tr.final_scores)
    return lockstep.GpuUnit(prefill_pos=tr.prefill_kept.copy(), evicted=tr.evicted.copy(), out=tr.out.copy(),
                            final_pos=fin, final_S=S)


def test_adaptive_checker_accepts_oracle_and_rejects_mistakes():
    from oracle import adaptive
    Q, K, V, ids = adaptive_case()
    P, hh, rc, R = 40, 4, 6, 16
    for T_ in (0.0, 0.5, 0.9, 2.0):                         # several choices
        tr = adaptive.run_unit(Q, K, V, ids, P, [0], [1, 2], hh, rc, 0.5, R, T_)
        g = adaptive_gpu_unit(tr)
        rep = lockstep.check_adaptive(Q, K, V, ids, P, [0], [1, 2], hh, rc, 0.5, R, T_, g, tr.choice)
        assert rep.ok and rep.adopted == 0, (T_, rep.failures)
    # a choice that skips a composite reaching the threshold
    tr = adaptive.run_unit(Q, K, V, ids, P, [0], [1, 2], hh, rc, 0.5, R, 0.0)
    assert tr.choice == adaptive.C_SPECIAL
    tr3 = adaptive.run_unit(Q, K, V, ids, P, [0], [1, 2], hh, rc, 0.5, R, 2.0)
    rep = lockstep.check_adaptive(Q, K, V, ids, P, [0], [1, 2], hh, rc, 0.5, R, 0.0, adaptive_gpu_unit(tr3), 5)
    assert not rep.ok
    # a wrong victim under the frequent+local composite (threshold = its recovery, so it is chosen)
    rec = tr3.recoveries
    assert rec[3] < rec[4]
    T4 = rec[4]
    trl = adaptive.run_unit(Q, K, V, ids, P, [0], [1, 2], hh, rc, 0.5, R, T4)
    assert trl.choice == adaptive.C_LOCAL
    g = adaptive_gpu_unit(trl)
    assert lockstep.check_adaptive(Q, K, V, ids, P, [0], [1, 2], hh, rc, 0.5, R, T4, g, 4).ok
    s = int(np.flatnonzero(trl.evicted >= 0)[2])
    bad = next(int(j) for j in trl.prefill_kept if int(j) != int(trl.evicted[s]) and ids[j] not in (0, 1, 2)
               and int(j) < P - rc)
    g.evicted[s] = bad
    assert not lockstep.check_adaptive(Q, K, V, ids, P, [0], [1, 2], hh, rc, 0.5, R, T4, g, 4).ok
    # an in-band choice: the threshold a hair above C4's recovery makes C5 the oracle's choice,
    # and C4 is then accepted (adopted) as within the recovery band
    rep = lockstep.check_adaptive(Q, K, V, ids, P, [0], [1, 2], hh, rc, 0.5, R, T4 + 1e-7, adaptive_gpu_unit(trl), 4)
    assert rep.adopted == 1 and not any("profile" in f for f in rep.failures)


def test_checkers_follow_the_cache_copy():
    """With a lossy cache copy (4-bit rows) the checkers accept the run made from
    that copy and reject the full-precision run, whose outputs differ."""
    from oracle import persistence, quant
    rng = np.random.default_rng(21)
    P, T, d, hh, r, w = 40, 20, 32, 6, 6, 16
    Q, K, V = (rng.standard_normal((P + T, d)) for _ in range(3))
    Kc, Vc = quant.roundtrip(K), quant.roundtrip(V)
    tq = h2o.run_unit(Q, K, V, P, hh, r, 0.3, Kc=Kc, Vc=Vc)
    tf = h2o.run_unit(Q, K, V, P, hh, r, 0.3)
    for tr, ok in ((tq, True), (tf, False)):
        g = lockstep.GpuUnit(prefill_pos=tr.prefill_kept.copy(), evicted=tr.evicted.copy(),
                             out=tr.out.copy(), final_pos=tr.final.pos.copy(),
                             prefill_S=tr.prefill_scores.copy(), final_S=tr.final.S.copy())
        assert lockstep.check_h2o(Q, K, V, P, hh, r, 0.3, g, Kc=Kc, Vc=Vc).ok == ok
    pq = persistence.run_unit(Q, K, V, P, hh, r, w, 0.3, Kc=Kc, Vc=Vc)
    pf = persistence.run_unit(Q, K, V, P, hh, r, w, 0.3)
    assert lockstep.check_persist(Q, K, V, P, hh, r, w, 0.3, persist_gpu_unit(pq, P), Kc=Kc, Vc=Vc).ok
    assert not lockstep.check_persist(Q, K, V, P, hh, r, w, 0.3, persist_gpu_unit(pf, P), Kc=Kc, Vc=Vc).ok


def test_hash_checker_follows_the_cache_copy():
    from oracle import quant
    rng = np.random.default_rng(23)
    N, P, d, B = 60, 40, 32, 16
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    W = rng.standard_normal((d, 32))
    Kc, Vc = quant.roundtrip(K), quant.roundtrip(V)
    for kc, vc, ok in ((Kc, Vc, True), (None, None, False)):
        tr = hashevict.run_unit(Q, K, V, W, P, B, 0.3, Kc=kc, Vc=vc)
        g = lockstep.GpuUnit(prefill_pos=tr.prefill_kept, evicted=tr.evicted.copy(), out=tr.out,
                             final_pos=tr.final_kept, prefill_S=None, final_S=None)
        assert lockstep.check_hash(Q, K, V, W, P, B, 0.3, g, Kc=Kc, Vc=Vc).ok == ok
