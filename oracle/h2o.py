"""H2O heavy-hitter eviction, in float64, step by step.

Test infrastructure only (see the package docstring).

Method, as the H2O page states it ([H2O], "提案手法" / proposed method and the
motivation list): a few tokens (heavy hitters) collect most of the attention;
the cache is kept small by a cheap dynamic greedy eviction driven by each
decode step's local attention statistics, balancing recency against
relevance.  The Scissorhands page ([SH], Abstract) states the same loop as a
cache held at a fixed budget that keeps the tokens that mattered.

Readings where the pages are silent (each one is listed in the design notes):

* score of a kept token = the sum of the softmax weights it has received from
  every query that saw it (prompt rows at prefill, then one per decode step),
  its own step included;
* prefill: the causal softmax of the prompt is formed once and its column sums
  are the scores; the kept set is the recent window [P - r, P) plus the
  ``heavy`` highest-scoring earlier positions;
* decode at position t: the query attends over the kept tokens plus the new
  token t, each weight is added to its token's score, and if that leaves more
  than heavy + recent tokens, the token with the lowest score among those not
  in the recent window (t - r, t] is evicted;
* one total order for every choice: lowest score first, then oldest position;
  equivalently the prefill top-k keeps the newer position on equal scores.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .attention import attend, causal_attention, causal_weights


@dataclass
class Cache:
    """Kept positions and their accumulated scores (aligned arrays)."""
    pos: np.ndarray                      # int64
    S: np.ndarray                        # float64


def prefill_column_scores(Q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """c_j = sum over prompt rows i >= j of the causal softmax weight p[i, j].

    [H2O] proposed method: accumulated local attention statistics; at prefill
    every prompt query contributes its row of weights.
    """
    return causal_weights(Q, K, scale).sum(axis=0)


def prefill_select(c: np.ndarray, heavy: int, recent: int) -> np.ndarray:
    """Positions kept after a prompt of length P = len(c), ascending.

    If P <= heavy + recent every position is kept.  Otherwise: the recent
    window [P - recent, P) plus the ``heavy`` positions of [0, P - recent) that
    rank highest by (score, position) -- equal scores keep the newer one.
    [H2O] proposed method (greedy on scores) and motivation (recency vs
    relevance).
    """
    P = len(c)
    if P <= heavy + recent:
        return np.arange(P, dtype=np.int64)
    candidates = range(0, P - recent)
    ranked = sorted(candidates, key=lambda j: (c[j], j), reverse=True)
    heavy_kept = sorted(ranked[:heavy])
    return np.array(heavy_kept + list(range(P - recent, P)), dtype=np.int64)


def prefill(Q: np.ndarray, K: np.ndarray, heavy: int, recent: int, scale: float):
    """Returns (cache, c): the kept positions with S_j = c_j, and all column scores."""
    c = prefill_column_scores(Q, K, scale)
    kept = prefill_select(c, heavy, recent)
    return Cache(kept, c[kept].copy()), c


def attend_step(cache: Cache, t: int, q: np.ndarray, K_all: np.ndarray, V_all: np.ndarray,
                scale: float, Kc: Optional[np.ndarray] = None, Vc: Optional[np.ndarray] = None):
    """Attention of the step-t query over the kept tokens plus token t itself.

    Returns (out [d], A, S_A): A = kept positions followed by t, and S_A the
    scores after this step's weights are added (S_t = its own weight).
    Kept tokens read what a cache slot holds (Kc / Vc, by position: the full
    sequences unless the cache stores a lossy format); token t is the step's
    own input, at full precision.
    """
    A = np.append(cache.pos, t).astype(np.int64)
    Kc = K_all if Kc is None else Kc
    Vc = V_all if Vc is None else Vc
    Ks = np.vstack([Kc[cache.pos], K_all[t:t + 1]])
    Vs = np.vstack([Vc[cache.pos], V_all[t:t + 1]])
    p, out = attend(q, Ks, Vs, scale)
    S_A = np.append(cache.S, 0.0) + p
    return out, A, S_A


def h2o_candidates(A: np.ndarray, t: int, recent: int) -> np.ndarray:
    """Indices into A of the positions outside the recent window (t - recent, t]."""
    return np.flatnonzero(A <= t - recent)


def h2o_victim(A: np.ndarray, S_A: np.ndarray, t: int, recent: int) -> int:
    """Index into A of the token to evict: lowest score, then oldest position."""
    cand = h2o_candidates(A, t, recent)
    return int(min(cand, key=lambda i: (S_A[i], A[i])))


def remove(A: np.ndarray, S_A: np.ndarray, idx: Optional[int]) -> Cache:
    if idx is None:
        return Cache(A, S_A)
    keep = np.ones(len(A), dtype=bool)
    keep[idx] = False
    return Cache(A[keep], S_A[keep])


@dataclass
class Trajectory:
    prefill_kept: np.ndarray
    prefill_scores: np.ndarray           # S of prefill_kept
    column_scores: np.ndarray            # c over the whole prompt
    out: np.ndarray                      # [T, d]
    evicted: np.ndarray                  # [T] position or -1
    evicted_score: np.ndarray            # [T] score at eviction or nan
    final: Cache
    prompt_out: Optional[np.ndarray] = None


def run_unit(Q_all: np.ndarray, K_all: np.ndarray, V_all: np.ndarray, P: int,
             heavy: int, recent: int, scale: float, steps: Optional[int] = None,
             want_prompt_out: bool = False, Kc: Optional[np.ndarray] = None,
             Vc: Optional[np.ndarray] = None) -> Trajectory:
    """Prefill on the first P positions, then decode positions P..P+steps-1.
    Kc / Vc: what cache slots read back per position (lossy cache formats)."""
    N = Q_all.shape[0]
    T = N - P if steps is None else steps
    budget = heavy + recent
    cache, c = prefill(Q_all[:P], K_all[:P], heavy, recent, scale)
    kept0, S0 = cache.pos.copy(), cache.S.copy()
    prompt_out = None
    if want_prompt_out:
        _, prompt_out = causal_attention(Q_all[:P], K_all[:P], V_all[:P], scale)
    outs, ev, evs = [], [], []
    for t in range(P, P + T):
        o, A, S_A = attend_step(cache, t, Q_all[t], K_all, V_all, scale, Kc, Vc)
        outs.append(o)
        if len(A) > budget:
            i = h2o_victim(A, S_A, t, recent)
            ev.append(int(A[i])); evs.append(float(S_A[i]))
            cache = remove(A, S_A, i)
        else:
            ev.append(-1); evs.append(float("nan"))
            cache = Cache(A, S_A)
    d = V_all.shape[1]
    return Trajectory(kept0, S0, c, np.array(outs).reshape(T, d), np.array(ev, dtype=np.int64),
                      np.array(evs), cache, prompt_out)
