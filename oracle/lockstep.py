"""Lockstep replay of one unit against a GPU run's logs.

Test infrastructure only (see the package docstring).

The oracle decides every eviction itself from its own float64 arithmetic on
the shared inputs.  The GPU's logged choice is compared with it:

* equal: continue;
* different but inside the near-tie band (the GPU's victim scores within a
  relative 1e-6 of the oracle's lowest candidate; for HashEvict, the GPU's
  victim is at the same maximal Hamming distance): accepted and counted, and
  the oracle continues from the GPU's choice;
* otherwise: a failure is recorded, and the oracle still continues from the
  GPU's choice so later steps stay comparable.

At the prompt the GPU's kept set is accepted if it has the right size, holds
the recent window, holds every candidate scoring above c_thr (1 + band) and
none scoring below c_thr (1 - band), where c_thr is the heavy-th largest
candidate score.

Tolerances: attention output per (unit, step) max|o_gpu - o_ref| <=
2e-3 max|o_ref|; accumulated scores |S_gpu - S_ref| <= 1e-5 S_ref per kept
slot; kept sets compared as sets of positions.

Persistence counts are integers decided by comparing a weight with 1/|A|;
the oracle flags the bits whose weight lies within a relative 1e-5 of that
threshold as ambiguous, bounds each count between its value with those bits
clear and set, and accepts a GPU choice that some setting of them explains.
The GPU's exported histories must equal the oracle's on every unambiguous
bit; at the prompt the oracle then takes the GPU's ambiguous bits, so the
replay continues from the GPU's state.

Profiled (adaptive) units: the GPU's composite choice is accepted if every
composite it passed over recovers less than threshold + 1e-5 and the chosen
one at least threshold - 1e-5 (recoveries are sums of float32 weights); the
replay then follows the GPU's choice with the H2O tie band for the frequent
part, protected tokens exact.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import adaptive, fastgen, h2o, hashevict, persistence
from .attention import attend, causal_attention

TIE_BAND = 1e-6
SCORE_RTOL = 1e-5
OUT_RTOL = 2e-3


@dataclass
class GpuUnit:
    """What the GPU run exported for one unit (positions as ints, scores float64)."""
    prefill_pos: np.ndarray              # kept positions after prefill (any order)
    evicted: np.ndarray                  # [T] position evicted at each step, -1 for none
    out: np.ndarray                      # [T, d]
    final_pos: np.ndarray                # kept positions after the last step (any order)
    prefill_S: Optional[np.ndarray] = None   # scores aligned with prefill_pos (H2O family)
    final_S: Optional[np.ndarray] = None     # scores aligned with final_pos (H2O family)
    prompt_out: Optional[np.ndarray] = None  # [P, d]


@dataclass
class UnitReport:
    failures: List[str] = field(default_factory=list)
    adopted: int = 0                     # near-ties where the GPU's in-band choice was adopted
    decisions: int = 0
    max_out_rel: float = 0.0
    max_prompt_out_rel: float = 0.0
    max_score_rel: float = 0.0
    min_gap: float = float("inf")        # smallest relative gap between the two lowest candidates
    gaps: List[float] = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return not self.failures

    def merge(self, o: "UnitReport", tag: str = "") -> None:
        self.failures += [f"{tag}{f}" for f in o.failures]
        self.adopted += o.adopted
        self.decisions += o.decisions
        self.max_out_rel = max(self.max_out_rel, o.max_out_rel)
        self.max_prompt_out_rel = max(self.max_prompt_out_rel, o.max_prompt_out_rel)
        self.max_score_rel = max(self.max_score_rel, o.max_score_rel)
        self.min_gap = min(self.min_gap, o.min_gap)
        self.gaps += o.gaps


def _out_rel(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    den = float(np.max(np.abs(o_ref)))
    num = float(np.max(np.abs(np.asarray(o_gpu, dtype=np.float64) - o_ref)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def _check_out(rep: UnitReport, step: int, o_gpu, o_ref) -> None:
    e = _out_rel(o_gpu, o_ref)
    rep.max_out_rel = max(rep.max_out_rel, e)
    if not e <= OUT_RTOL:
        rep.failures.append(f"step {step}: output rel err {e:.3e} > {OUT_RTOL}")


def _check_prompt_out(rep: UnitReport, gpu: GpuUnit, Q, K, V, P, scale) -> None:
    if gpu.prompt_out is None:
        return
    _, ref = causal_attention(Q[:P], K[:P], V[:P], scale)
    for i in range(P):
        e = _out_rel(gpu.prompt_out[i], ref[i])
        rep.max_prompt_out_rel = max(rep.max_prompt_out_rel, e)
        if not e <= OUT_RTOL:
            rep.failures.append(f"prompt row {i}: output rel err {e:.3e}")
            return


def _check_scores(rep: UnitReport, where: str, pos_gpu, S_gpu, ref_pos, ref_S) -> None:
    if S_gpu is None:
        return
    ref = dict(zip((int(p) for p in ref_pos), ref_S))
    for p, s in zip(pos_gpu, S_gpu):
        r = ref.get(int(p))
        if r is None:
            continue                      # set mismatch is reported separately
        e = abs(float(s) - r) / r if r > 0 else (0.0 if s == r else float("inf"))
        rep.max_score_rel = max(rep.max_score_rel, e)
        if not e <= SCORE_RTOL:
            rep.failures.append(f"{where}: score of position {int(p)} rel err {e:.3e}")


def check_prefill_set(rep: UnitReport, c: np.ndarray, gpu_pos: np.ndarray, heavy: int,
                       recent: int) -> np.ndarray:
    """Validates the GPU's prompt kept set in the tie band; returns the set to continue from."""
    P = len(c)
    gpu = np.unique(np.asarray(gpu_pos, dtype=np.int64))
    if len(gpu) != len(gpu_pos):
        rep.failures.append("prefill: duplicate positions")
    ref = h2o.prefill_select(c, heavy, recent)
    if np.array_equal(gpu, ref):
        return ref
    if P <= heavy + recent:
        rep.failures.append("prefill: kept set differs with P <= budget")
        return gpu
    ok = len(gpu) == heavy + recent and set(range(P - recent, P)) <= set(gpu.tolist())
    cand_gpu = gpu[gpu < P - recent]
    ranked = np.sort(c[: P - recent])[::-1]
    thr = ranked[heavy - 1] if heavy > 0 else np.inf
    above = np.flatnonzero(c[: P - recent] > thr * (1 + TIE_BAND))
    below = set(np.flatnonzero(c[: P - recent] < thr * (1 - TIE_BAND)).tolist())
    ok = ok and set(above.tolist()) <= set(cand_gpu.tolist())
    ok = ok and not (set(cand_gpu.tolist()) & below)
    if ok:
        rep.adopted += 1
    else:
        rep.failures.append("prefill: kept set outside the near-tie band")
    return gpu


def accept_h2o_victim(A: np.ndarray, S_A: np.ndarray, cand: np.ndarray, i_ref: int, g: int) -> bool:
    """True iff position g is an admissible victim whose score is within the
    relative tie band of the oracle's lowest candidate score S_A[i_ref]."""
    where = np.flatnonzero(A == g)
    return (len(where) == 1 and int(where[0]) in set(int(x) for x in cand)
            and S_A[where[0]] <= S_A[i_ref] * (1 + TIE_BAND))


def check_h2o(Q, K, V, P: int, heavy: int, recent: int, scale: float, gpu: GpuUnit,
              steps: Optional[int] = None, Kc=None, Vc=None) -> UnitReport:
    """H2O family (also FastGen frequency+local heads).  Kc / Vc: cache slot
    contents per position for lossy cache formats."""
    rep = UnitReport()
    T = len(gpu.evicted) if steps is None else steps
    budget = heavy + recent
    c = h2o.prefill_column_scores(Q[:P], K[:P], scale)
    kept = check_prefill_set(rep, c, gpu.prefill_pos, heavy, recent)
    _check_scores(rep, "prefill", gpu.prefill_pos, gpu.prefill_S, kept, c[kept])
    _check_prompt_out(rep, gpu, Q, K, V, P, scale)
    cache = h2o.Cache(kept.copy(), c[kept].copy())
    for s in range(T):
        t = P + s
        o, A, S_A = h2o.attend_step(cache, t, Q[t], K, V, scale, Kc, Vc)
        _check_out(rep, s, gpu.out[s], o)
        g = int(gpu.evicted[s])
        if len(A) <= budget:
            if g != -1:
                rep.failures.append(f"step {s}: evicted {g} with the cache under budget")
            cache = h2o.Cache(A, S_A)
            continue
        rep.decisions += 1
        cand = h2o.h2o_candidates(A, t, recent)
        i_ref = h2o.h2o_victim(A, S_A, t, recent)
        sc = np.sort(S_A[cand])
        if len(sc) > 1:
            gap = (sc[1] - sc[0]) / sc[0]
            rep.gaps.append(float(gap))
            rep.min_gap = min(rep.min_gap, float(gap))
        if g == int(A[i_ref]):
            cache = h2o.remove(A, S_A, i_ref)
            continue
        where = np.flatnonzero(A == g)
        if accept_h2o_victim(A, S_A, cand, i_ref, g):
            rep.adopted += 1
        else:
            rep.failures.append(f"step {s}: GPU evicted {g}, oracle {int(A[i_ref])} "
                                f"(S {S_A[where[0]] if len(where) else float('nan'):.9g} vs "
                                f"{S_A[i_ref]:.9g})")
        cache = h2o.remove(A, S_A, int(where[0])) if len(where) == 1 else h2o.remove(A, S_A, i_ref)
    if not np.array_equal(np.sort(np.asarray(gpu.final_pos, dtype=np.int64)), np.sort(cache.pos)):
        rep.failures.append("final kept set differs")
    _check_scores(rep, "final", gpu.final_pos, gpu.final_S, cache.pos, cache.S)
    return rep


def check_positional(tr: fastgen.Trajectory, gpu: GpuUnit, Q, K, V, P, scale) -> UnitReport:
    """FULL / LOCAL / SPECIAL heads: choices are fixed by position or token id, so the
    kept sets and the eviction log must match exactly."""
    rep = UnitReport()
    if not np.array_equal(np.sort(np.asarray(gpu.prefill_pos, dtype=np.int64)), np.sort(tr.prefill_kept)):
        rep.failures.append("prefill kept set differs")
    _check_prompt_out(rep, gpu, Q, K, V, P, scale)
    T = len(tr.evicted)
    for s in range(T):
        _check_out(rep, s, gpu.out[s], tr.out[s])
        if int(gpu.evicted[s]) != int(tr.evicted[s]):
            rep.failures.append(f"step {s}: evicted {int(gpu.evicted[s])} vs {int(tr.evicted[s])}")
    if not np.array_equal(np.sort(np.asarray(gpu.final_pos, dtype=np.int64)), np.sort(tr.final_kept)):
        rep.failures.append("final kept set differs")
    return rep


def check_fastgen(policy: int, Q, K, V, P, scale, gpu: GpuUnit, *, heavy=0, recent=0, ids=None,
                  keep_ids=(), steps=None) -> UnitReport:
    if policy == fastgen.H2O:
        return check_h2o(Q, K, V, P, heavy, recent, scale, gpu, steps)
    T = len(gpu.evicted) if steps is None else steps
    tr = fastgen.run_unit(policy, Q, K, V, P, scale, heavy=heavy, recent=recent, ids=ids,
                          keep_ids=keep_ids, steps=T)
    return check_positional(tr, gpu, Q, K, V, P, scale)


def check_hash(Q, K, V, Wp, P: int, B: int, scale: float, gpu: GpuUnit, steps: Optional[int] = None,
               qsk=None, ksk=None, Kc=None, Vc=None) -> UnitReport:
    """HashEvict: integer distances, so choices must match; at equal maximal distance any
    maximiser is accepted (and counted) -- the GPU uses the same oldest-first order,
    so none is expected.  Kc / Vc: cache slot contents per position (lossy formats);
    HashEvict attends the cache after the insertion, token t included."""
    Kc = K if Kc is None else Kc
    Vc = V if Vc is None else Vc
    rep = UnitReport()
    T = len(gpu.evicted) if steps is None else steps
    if qsk is None:
        qsk = hashevict.sketches(Q[:P + T], Wp)
    if ksk is None:
        ksk = hashevict.sketches(K[:P + T], Wp)
    kept = hashevict.replay_prompt(qsk, ksk, P, B)
    if not np.array_equal(np.sort(np.asarray(gpu.prefill_pos, dtype=np.int64)), np.sort(kept)):
        rep.failures.append("prefill (replay) kept set differs")
        kept = np.asarray(gpu.prefill_pos, dtype=np.int64)
    _check_prompt_out(rep, gpu, Q, K, V, P, scale)
    cache = list(int(x) for x in kept)
    for s in range(T):
        t = P + s
        g = int(gpu.evicted[s])
        if len(cache) >= B:
            rep.decisions += 1
            arr = np.array(cache, dtype=np.int64)
            v = hashevict.farthest(int(qsk[t]), arr, ksk)
            if g != cache[v]:
                h = hashevict.hamming(np.uint64(qsk[t]), ksk[arr])
                w = np.flatnonzero(arr == g)
                if len(w) == 1 and h[w[0]] == h.max():
                    rep.adopted += 1
                    v = int(w[0])
                else:
                    rep.failures.append(f"step {s}: GPU evicted {g}, oracle {cache[v]}")
                    if len(w) == 1:
                        v = int(w[0])
            cache[v] = t
        else:
            if g != -1:
                rep.failures.append(f"step {s}: evicted {g} under budget")
            cache.append(t)
        A = np.array(cache, dtype=np.int64)
        _check_out(rep, s, gpu.out[s], attend(Q[t], Kc[A], Vc[A], scale)[1])
    if not np.array_equal(np.sort(np.asarray(gpu.final_pos, dtype=np.int64)), np.sort(np.array(cache))):
        rep.failures.append("final kept set differs")
    return rep


def _as_bits(x) -> np.ndarray:
    """Histories exported in the float64 score array: the raw 64-bit patterns."""
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64)).view(np.uint64)


def _count_bounds(hist: np.ndarray, amb: np.ndarray):
    lo = persistence.count(hist & ~amb)
    hi = persistence.count(hist | amb)
    return lo, hi


def _check_history_bits(rep: UnitReport, where: str, pos, gpu_bits, ref_pos, ref_hist, ref_amb) -> None:
    ref = {int(p): (int(h), int(a)) for p, h, a in zip(ref_pos, ref_hist, ref_amb)}
    for p, g in zip(pos, gpu_bits):
        r = ref.get(int(p))
        if r is None:
            continue                      # set mismatch is reported separately
        if (int(g) ^ r[0]) & ~r[1] & ((1 << 64) - 1):
            rep.failures.append(f"{where}: history of position {int(p)} {int(g):#x} vs {r[0]:#x} "
                                f"(ambiguous {r[1]:#x})")


def check_persist(Q, K, V, P: int, heavy: int, recent: int, window: int, scale: float, gpu: GpuUnit,
                  steps: Optional[int] = None, Kc=None, Vc=None) -> UnitReport:
    """Persistence-count eviction (Scissorhands reading)."""
    rep = UnitReport()
    T = len(gpu.evicted) if steps is None else steps
    budget = heavy + recent
    hist, amb = persistence.prefill_histories(Q[:P], K[:P], scale, window)
    gpos = np.asarray(gpu.prefill_pos, dtype=np.int64)
    ref = h2o.prefill_select(persistence.count(hist).astype(np.float64), heavy, recent)
    if len(np.unique(gpos)) != len(gpos):
        rep.failures.append("prefill: duplicate positions")
    if not np.array_equal(np.sort(gpos), ref):
        ok = P > budget and len(gpos) == budget and set(range(P - recent, P)) <= set(gpos.tolist())
        lo, hi = _count_bounds(hist, amb)
        kept_heavy = [int(j) for j in gpos if j < P - recent]
        dropped = sorted(set(range(P - recent)) - set(kept_heavy))
        if ok and kept_heavy and dropped:
            weakest = min((int(hi[j]), j) for j in kept_heavy)
            strongest = max((int(lo[k]), k) for k in dropped)
            ok = strongest < weakest
        if ok:
            rep.adopted += 1
        else:
            rep.failures.append("prefill: kept set not explained by the ambiguous bits")
    kept = np.sort(gpos)
    k_hist, k_amb = hist[kept].copy(), amb[kept].copy()
    if gpu.prefill_S is not None:
        order = np.argsort(gpos)
        gbits = _as_bits(gpu.prefill_S)[order]
        _check_history_bits(rep, "prefill", kept, gbits, kept, k_hist, k_amb)
        k_hist = (k_hist & ~k_amb) | (gbits & k_amb)
        k_amb = np.zeros_like(k_amb)
    _check_prompt_out(rep, gpu, Q, K, V, P, scale)
    cache = persistence.Cache(kept, k_hist, k_amb)
    for s in range(T):
        t = P + s
        o, A, hA, aA, _ = persistence.attend_step(cache, t, Q[t], K, V, scale, window, Kc, Vc)
        _check_out(rep, s, gpu.out[s], o)
        g = int(gpu.evicted[s])
        if len(A) <= budget:
            if g != -1:
                rep.failures.append(f"step {s}: evicted {g} with the cache under budget")
            cache = persistence.Cache(A, hA, aA)
            continue
        rep.decisions += 1
        i_ref = persistence.victim(A, hA, t, recent)
        if g == int(A[i_ref]):
            cache = persistence.remove(A, hA, aA, i_ref)
            continue
        where = np.flatnonzero(A == g)
        cand = persistence.candidates(A, t, recent)
        lo, hi = _count_bounds(hA, aA)
        ok = len(where) == 1 and int(where[0]) in set(int(x) for x in cand)
        if ok:
            gi = int(where[0])
            ok = not any((int(hi[k]), int(A[k])) < (int(lo[gi]), g) for k in cand if k != gi)
        if ok:
            rep.adopted += 1
        else:
            rep.failures.append(f"step {s}: GPU evicted {g}, oracle {int(A[i_ref])}")
        cache = persistence.remove(A, hA, aA, int(where[0]) if len(where) == 1 else i_ref)
    if not np.array_equal(np.sort(np.asarray(gpu.final_pos, dtype=np.int64)), np.sort(cache.pos)):
        rep.failures.append("final kept set differs")
    if gpu.final_S is not None:
        _check_history_bits(rep, "final", gpu.final_pos, _as_bits(gpu.final_S), cache.pos, cache.hist, cache.amb)
    return rep


RECOVERY_BAND = 1e-5


def check_adaptive(Q, K, V, ids, P: int, special, punct, heavy: int, recent: int, scale: float, rows: int,
                   threshold: float, gpu: GpuUnit, gpu_choice: int, steps: Optional[int] = None) -> UnitReport:
    """FastGen profiling + the chosen composite, in lockstep."""
    rep = UnitReport()
    T = len(gpu.evicted) if steps is None else steps
    comps = adaptive.composites(special, punct, heavy, recent)
    k_ref, rec = adaptive.profile(Q[:P], K[:P], ids, comps, scale, rows, threshold)
    g = int(gpu_choice)
    if g != k_ref:
        passed = [j for j in (1, 2, 3, 4) if j < g]
        ok = g in comps and all(rec.get(j, 0.0) < threshold + RECOVERY_BAND for j in passed)
        ok = ok and (g == adaptive.C_FULL or rec.get(g, 0.0) >= threshold - RECOVERY_BAND)
        if ok:
            rep.adopted += 1
        else:
            rep.failures.append(f"profile: GPU chose C{g}, oracle C{k_ref} (recoveries {rec})")
            if g not in comps:
                return rep
    comp = comps[g]
    c = h2o.prefill_column_scores(Q[:P], K[:P], scale)
    ref = adaptive.prompt_kept(comp, c, ids, P)
    gpos = np.sort(np.asarray(gpu.prefill_pos, dtype=np.int64))
    if not np.array_equal(gpos, ref):
        prot = {j for j in range(P) if int(ids[j]) in comp.protected}
        free = [j for j in range(P) if j not in prot]
        window = {j for j in free if j >= P - comp.recent}
        older = [j for j in free if j < P - comp.recent]
        quota = comp.heavy + comp.recent - len(window)
        got = set(gpos.tolist())
        ok = not comp.full and len(free) > comp.heavy + comp.recent and (prot | window) <= got
        heavy_got = [j for j in got if j in set(older)]
        ok = ok and len(heavy_got) == quota and len(got) == len(prot) + len(window) + quota
        if ok and quota > 0:
            ranked = np.sort(c[older])[::-1]
            thr = ranked[quota - 1]
            ok = all(j in got for j in older if c[j] > thr * (1 + TIE_BAND))
            ok = ok and not any(j in got for j in older if c[j] < thr * (1 - TIE_BAND))
        if ok:
            rep.adopted += 1
        else:
            rep.failures.append("prefill: kept set outside the near-tie band")
    kept = gpos
    S = c[kept].copy()
    _check_prompt_out(rep, gpu, Q, K, V, P, scale)
    for s_ in range(T):
        t = P + s_
        A = np.append(kept, t).astype(np.int64)
        p, o = attend(Q[t], K[A], V[A], scale)
        _check_out(rep, s_, gpu.out[s_], o)
        S_A = np.append(S, 0.0) + p
        gv = int(gpu.evicted[s_])
        free = np.array([int(ids[j]) not in comp.protected for j in A])
        if comp.full or int(ids[t]) in comp.protected or free.sum() <= comp.heavy + comp.recent:
            if gv != -1:
                rep.failures.append(f"step {s_}: evicted {gv}, none expected")
            kept, S = A, S_A
            continue
        rep.decisions += 1
        cand = np.array([i for i in range(len(A)) if free[i] and A[i] <= t - comp.recent], dtype=np.int64)
        i_ref = int(min(cand, key=lambda i: (S_A[i], A[i])))
        where = np.flatnonzero(A == gv)
        if gv != int(A[i_ref]):
            if accept_h2o_victim(A, S_A, cand, i_ref, gv):
                rep.adopted += 1
            else:
                rep.failures.append(f"step {s_}: GPU evicted {gv}, oracle {int(A[i_ref])}")
        v = int(where[0]) if len(where) == 1 else i_ref
        keep = np.ones(len(A), dtype=bool)
        keep[v] = False
        kept, S = A[keep], S_A[keep]
    if not np.array_equal(np.sort(np.asarray(gpu.final_pos, dtype=np.int64)), np.sort(kept)):
        rep.failures.append("final kept set differs")
    if gpu.final_S is not None and not comp.full:
        gmap = {int(p_): float(v_) for p_, v_ in zip(gpu.final_pos, gpu.final_S)}
        ref_S = {int(j): float(v_) for j, v_ in zip(kept, S)}
        free_pos = [int(j) for j in kept if int(ids[j]) not in comp.protected and int(j) in gmap]
        _check_scores(rep, "final", free_pos, [gmap[j] for j in free_pos], free_pos, [ref_S[j] for j in free_pos])
    return rep
