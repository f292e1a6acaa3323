"""FastGen's attention profiling and its hybrid (composite) policies, in float64.

Test infrastructure only (see the package docstring).

What the FastGen page states ([FG] "提案手法" / proposed method and "主な発見"):
a lightweight profiling step reads the attention map and assigns every head a
compression policy; the policies are combined greedily, the most effective
first -- special tokens, then punctuation, then frequent tokens, then the
local window -- which is the order that gave the best quality and compression;
heads that attend broadly keep the standard full cache.  The page gives no
formula for the profile, no threshold and no budgets, so the rest is a
reading (each one is listed in the design notes):

* composites, in greedy order: C1 = special, C2 = C1 + punctuation,
  C3 = C2 + frequent, C4 = C3 + local; C5 = the full cache;
* a composite keeps the tokens whose id is in its id set for good
  ("protected"); every other token belongs to an H2O cache of ``heavy``
  frequent slots and a ``recent`` local window (C1, C2: no slots, so an
  unprotected new token leaves at once; C3: no window);
* its kept set at the end of a prompt of P tokens: the protected tokens, the
  unprotected tokens of [P - recent, P), and, up to heavy + recent unprotected
  tokens in all, the unprotected earlier tokens with the largest column
  scores of the causal softmax (the newer first on equal scores) -- the state
  the decode rule below holds, where protected tokens in the window use no
  budget;
* decode at position t: the query attends the kept tokens plus t, every
  weight is added to its token's score; a protected t is kept; otherwise, if
  more than heavy + recent unprotected tokens remain, the unprotected token
  with the lowest score outside (t - recent, t] leaves, the oldest first;
* profile: the last R = min(rows, P) prompt rows; the recovery of a composite
  is the mean over those rows of the softmax mass the row gives to the
  composite's end-of-prompt kept set (keys up to the row); the first
  composite whose recovery reaches the threshold is chosen, else C5.  One
  profile per (sequence, head), from that sequence's prompt.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

from .attention import attend, causal_attention, causal_weights

C_SPECIAL, C_PUNCT, C_FREQUENT, C_LOCAL, C_FULL = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Composite:
    """A hybrid policy: protected ids, H2O slots for the rest, or the full cache."""
    protected: frozenset
    heavy: int
    recent: int
    full: bool = False


def composites(special: Sequence[int], punct: Sequence[int], heavy: int, recent: int):
    """C1..C5 in the page's greedy order."""
    sp = frozenset(int(x) for x in special)
    spp = sp | frozenset(int(x) for x in punct)
    return {
        C_SPECIAL: Composite(sp, 0, 0),
        C_PUNCT: Composite(spp, 0, 0),
        C_FREQUENT: Composite(spp, heavy, 0),
        C_LOCAL: Composite(spp, heavy, recent),
        C_FULL: Composite(frozenset(), 0, 0, True),
    }


def prompt_kept(comp: Composite, c: np.ndarray, ids: np.ndarray, P: int) -> np.ndarray:
    """Kept positions (ascending) after a prompt of P tokens with column scores c."""
    if comp.full:
        return np.arange(P, dtype=np.int64)
    prot = [j for j in range(P) if int(ids[j]) in comp.protected]
    free = [j for j in range(P) if int(ids[j]) not in comp.protected]
    if len(free) <= comp.heavy + comp.recent:
        return np.arange(P, dtype=np.int64)
    window = [j for j in free if j >= P - comp.recent]
    older = [j for j in free if j < P - comp.recent]
    ranked = sorted(older, key=lambda j: (c[j], j), reverse=True)[:comp.heavy + comp.recent - len(window)]
    return np.array(sorted(prot + window + ranked), dtype=np.int64)


def recovery(p: np.ndarray, kept: np.ndarray, rows: int) -> float:
    """Mean over the last `rows` rows of p (a causal softmax) of the mass on `kept`."""
    P = p.shape[0]
    R = min(rows, P)
    mask = np.zeros(P, dtype=bool)
    mask[kept] = True
    return float(np.mean([p[i, : i + 1][mask[: i + 1]].sum() for i in range(P - R, P)]))


def profile(Q: np.ndarray, K: np.ndarray, ids: np.ndarray, comps, scale: float, rows: int,
            threshold: float) -> Tuple[int, dict]:
    """Returns (chosen composite index, {index: recovery}) for one prompt."""
    P = Q.shape[0]
    p = causal_weights(Q, K, scale)
    c = p.sum(axis=0)
    rec = {}
    for k in (C_SPECIAL, C_PUNCT, C_FREQUENT, C_LOCAL):
        rec[k] = recovery(p, prompt_kept(comps[k], c, ids, P), rows)
        if rec[k] >= threshold:
            return k, rec
    return C_FULL, rec


@dataclass
class Trajectory:
    choice: int
    recoveries: dict
    prefill_kept: np.ndarray
    prefill_scores: np.ndarray           # column scores of prefill_kept
    out: np.ndarray                      # [T, d]
    evicted: np.ndarray                  # [T] position or -1
    final_kept: np.ndarray
    final_scores: np.ndarray             # accumulated scores of final_kept (protected tokens too)
    protected_final: np.ndarray          # bool, aligned with final_kept
    prompt_out: Optional[np.ndarray] = None


def run_composite(comp: Composite, Q_all, K_all, V_all, ids, P: int, scale: float, steps=None):
    """Prefill + decode under one composite.  Returns (kept0, S0, out, evicted, kept, S)."""
    T = Q_all.shape[0] - P if steps is None else steps
    c = causal_weights(Q_all[:P], K_all[:P], scale).sum(axis=0)
    kept = prompt_kept(comp, c, ids, P)
    S = c[kept].copy()
    kept0, S0 = kept.copy(), S.copy()
    outs, ev = [], []
    for t in range(P, P + T):
        A = np.append(kept, t).astype(np.int64)
        p, o = attend(Q_all[t], K_all[A], V_all[A], scale)
        outs.append(o)
        S_A = np.append(S, 0.0) + p
        if comp.full or int(ids[t]) in comp.protected:
            kept, S = A, S_A
            ev.append(-1)
            continue
        free = np.array([int(ids[j]) not in comp.protected for j in A])
        if free.sum() <= comp.heavy + comp.recent:
            kept, S = A, S_A
            ev.append(-1)
            continue
        cand = [i for i in range(len(A)) if free[i] and A[i] <= t - comp.recent]
        v = min(cand, key=lambda i: (S_A[i], A[i]))
        ev.append(int(A[v]))
        keep = np.ones(len(A), dtype=bool)
        keep[v] = False
        kept, S = A[keep], S_A[keep]
    d = V_all.shape[1]
    return kept0, S0, np.array(outs).reshape(T, d), np.array(ev, dtype=np.int64), kept, S


def run_unit(Q_all, K_all, V_all, ids, P: int, special, punct, heavy: int, recent: int, scale: float,
             rows: int, threshold: float, steps=None, want_prompt_out=False) -> Trajectory:
    """Profile the prompt, choose the composite, then prefill and decode under it."""
    comps = composites(special, punct, heavy, recent)
    k, rec = profile(Q_all[:P], K_all[:P], ids, comps, scale, rows, threshold)
    kept0, S0, out, ev, kept, S = run_composite(comps[k], Q_all, K_all, V_all, ids, P, scale, steps)
    prot = np.array([int(ids[j]) in comps[k].protected for j in kept], dtype=bool)
    po = causal_attention(Q_all[:P], K_all[:P], V_all[:P], scale)[1] if want_prompt_out else None
    return Trajectory(k, rec, kept0, S0, out, ev, kept, S, prot, po)
