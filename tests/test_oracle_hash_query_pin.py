"""Pin of the HashEvict decision's operand: the current query's sketch (CPU only).

[HE] 要約 / original abstract: at each step the current query's binarised
projection is compared with every cached key's by Hamming distance, and the
farthest key is replaced before attention.  With the identity projection
(d = bits) a sketch is the sign pattern of the vector, so inputs can be built
whose decisions follow in closed form:

* every position gets a distinct key sketch;
* the query of each replacing position i (prompt i >= B, every decode step)
  has the bitwise complement of one scheduled cache member's sketch: that
  member is at distance `bits`, every other member (distinct sketch) closer,
  so it is the unique farthest key;
* the new token's own key sketch is the complement of a *different* cache
  member, so ranking by the new key's sketch would pick that one instead.

The schedule is drawn first and the expected kept sets and victims follow from
it by list bookkeeping alone (no distances).  Planted mistakes -- the new key's
sketch in place of the query's, or the previous position's query -- are fed to
the oracle through its sketch arguments and must break the closed form.
"""

import numpy as np
import pytest

from oracle import hashevict, lockstep


def _signs(sk: int, bits: int, rng) -> np.ndarray:
    """A vector whose coordinate b is positive iff bit b of sk is set (never 0)."""
    mag = 0.25 + rng.random(bits)
    sgn = np.array([1.0 if (sk >> b) & 1 else -1.0 for b in range(bits)])
    return sgn * mag


def build(bits: int, P: int, T: int, B: int, seed: int):
    """Inputs plus the closed-form schedule: (Q, K, V, W, kept after the prompt,
    victim per decode step, final kept set)."""
    rng = np.random.default_rng(seed)
    full = (1 << bits) - 1
    N = P + T
    ksk = [0] * N
    qsk = [0] * N
    used = set()

    def fresh():
        while True:
            s = int(rng.integers(0, 1 << 32)) | (int(rng.integers(0, 1 << 32)) << 32)
            s &= full
            if s not in used:
                used.add(s)
                return s

    # positions [0, B) enter without replacing anything (prompt, then decode if P < B)
    for j in range(min(B, N)):
        ksk[j] = fresh()
    cache = list(range(min(B, N)))
    victims = [-1] * max(0, min(B, N) - P)   # decode steps that only append
    for i in range(B, N):
        # scheduled victim: any member but the oldest when possible (so FIFO differs)
        order = sorted(cache)
        pick = order[1 + int(rng.integers(0, len(order) - 1))] if len(order) > 1 else order[0]
        qsk[i] = full ^ ksk[pick]
        # the new key's sketch aims at another member, and stays distinct from all
        others = [m for m in cache if m != pick]
        rng.shuffle(others)
        for w in others:
            cand = full ^ ksk[w]
            if cand not in used and cand != ksk[pick]:
                ksk[i] = cand
                used.add(cand)
                break
        else:
            ksk[i] = fresh()
        cache[cache.index(pick)] = i
        victims.append(pick)
    # queries of positions that replace nothing (i < B) are arbitrary
    for i in range(min(B, N)):
        qsk[i] = int(rng.integers(0, 1 << min(bits, 62)))
    # the cache right after the prompt follows from the prompt part of the
    # schedule; in slot order (each replacement takes its victim's slot) it
    # records the whole sequence of prompt victims
    kept_prompt = list(range(min(P, B)))
    for i, v in zip(range(B, P), victims[: max(0, P - B)]):
        kept_prompt[kept_prompt.index(v)] = i
    Q = np.stack([_signs(qsk[i], bits, rng) for i in range(N)])
    K = np.stack([_signs(ksk[i], bits, rng) for i in range(N)])
    V = rng.standard_normal((N, bits))
    W = np.eye(bits)
    dec_victims = victims[max(0, P - B):]
    assert len(dec_victims) == T
    return Q, K, V, W, kept_prompt, dec_victims, sorted(cache)


CASES = [(32, 40, 30, 12, 1), (32, 13, 25, 12, 2), (16, 30, 40, 9, 3), (64, 50, 20, 17, 4), (32, 64, 64, 32, 5),
         (32, 8, 30, 12, 6)]


@pytest.mark.parametrize("bits,P,T,B,seed", CASES)
def test_query_sketch_decides_in_closed_form(bits, P, T, B, seed):
    Q, K, V, W, kept0, dec_v, final = build(bits, P, T, B, seed)
    qsk = hashevict.sketches(Q, W)
    ksk = hashevict.sketches(K, W)
    # the construction holds: distinct key sketches
    assert len(set(ksk.tolist())) == P + T
    tr = hashevict.run_unit(Q, K, V, W, P, B, 0.2)
    assert tr.prefill_kept.tolist() == sorted(kept0)
    assert tr.evicted.tolist() == dec_v
    assert tr.final_kept.tolist() == final
    # the replay alone, slot by slot
    assert hashevict.replay_prompt(qsk, ksk, P, B).tolist() == kept0


def _mutants(qsk, ksk, P):
    """Sketch arguments that plant each mistake in the oracle's decisions."""
    prev = np.roll(qsk, 1)                   # position i ranks with q_{i-1}
    dec_key = qsk.copy()
    dec_key[P:] = ksk[P:]                    # decode ranks with the new key's sketch
    dec_prev = qsk.copy()
    dec_prev[P:] = qsk[P - 1:-1]             # decode ranks with the previous query
    return {"replay and decode use the new key": ksk, "replay and decode use q_{i-1}": prev,
            "decode uses the new key": dec_key, "decode uses q_{t-1}": dec_prev}


@pytest.mark.parametrize("bits,P,T,B,seed", CASES)
def test_planted_operand_mistakes_break_the_closed_form(bits, P, T, B, seed):
    Q, K, V, W, kept0, dec_v, final = build(bits, P, T, B, seed)
    qsk = hashevict.sketches(Q, W)
    ksk = hashevict.sketches(K, W)
    for name, qm in _mutants(qsk, ksk, P).items():
        tr = hashevict.run_unit(Q, K, V, W, P, B, 0.2, qsk=qm, ksk=ksk)
        caught = (tr.prefill_kept.tolist() != sorted(kept0) or tr.evicted.tolist() != dec_v
                  or tr.final_kept.tolist() != final)
        assert caught, f"planted mistake not caught: {name}"
    if P > B:
        # the replay alone: ranking by the new key's sketch or by q_{i-1}
        # changes the sequence of prompt victims
        assert hashevict.replay_prompt(ksk, ksk, P, B).tolist() != kept0
        assert hashevict.replay_prompt(np.roll(qsk, 1), ksk, P, B).tolist() != kept0


@pytest.mark.parametrize("bits,P,T,B,seed", CASES[:3])
def test_lockstep_checker_follows_the_query(bits, P, T, B, seed):
    """The lockstep checker accepts the closed-form log and rejects the log a
    key-ranked run would produce."""
    Q, K, V, W, kept0, dec_v, final = build(bits, P, T, B, seed)
    good = hashevict.run_unit(Q, K, V, W, P, B, 0.2)
    log = lockstep.GpuUnit(prefill_pos=np.array(sorted(kept0)), evicted=np.array(dec_v), out=good.out,
                           final_pos=np.array(final))
    rep = lockstep.check_hash(Q, K, V, W, P, B, 0.2, log)
    assert rep.ok, rep.failures[:3]
    # every farthest key is unique here, so nothing may need the tie band
    assert rep.adopted == 0 and rep.decisions == T - max(0, B - P)
    qsk = hashevict.sketches(Q, W)
    ksk = hashevict.sketches(K, W)
    bad = hashevict.run_unit(Q, K, V, W, P, B, 0.2, qsk=ksk, ksk=ksk)
    badlog = lockstep.GpuUnit(prefill_pos=bad.prefill_kept, evicted=bad.evicted, out=bad.out,
                              final_pos=bad.final_kept)
    assert not lockstep.check_hash(Q, K, V, W, P, B, 0.2, badlog).ok
    # right prompt, key-ranked decode: every such victim is at the largest
    # distance from the new key's sketch, so only a query-ranked band rejects it
    qdec = qsk.copy()
    qdec[P:] = ksk[P:]
    bad2 = hashevict.run_unit(Q, K, V, W, P, B, 0.2, qsk=qdec, ksk=ksk)
    assert bad2.prefill_kept.tolist() == sorted(kept0) and bad2.evicted.tolist() != dec_v
    badlog2 = lockstep.GpuUnit(prefill_pos=bad2.prefill_kept, evicted=bad2.evicted, out=bad2.out,
                               final_pos=bad2.final_kept)
    rep2 = lockstep.check_hash(Q, K, V, W, P, B, 0.2, badlog2)
    assert not rep2.ok and rep2.adopted == 0
