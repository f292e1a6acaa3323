"""Scissorhands-style persistence of importance, in float64, step by step.

Test infrastructure only (see the package docstring).

What the page states ([SH], Abstract): only pivotal tokens -- those that had
a substantial influence at one step -- will significantly influence later
steps; the system holds the KV cache at a fixed budget and keeps the pivotal
tokens with a higher probability.  The page gives no formula, threshold,
window or tie rule, so everything below the first sentence is a reading
(each one is listed in the design notes):

* a token is *pivotal* at a step if the softmax weight the step's query gives
  it is at least the uniform weight 1 / |A|, A being every key that query
  attends over (at prompt row i: the i + 1 keys 0..i; at decode step t: the
  kept tokens plus t);
* every kept token carries the pivotal bits of the last ``window`` steps that
  attended it (1 <= window <= 64): bit k is the step k steps before the
  latest one; its *persistence count* is the number of set bits;
* prefill: token j's bits come from the prompt rows i in [max(j, P - window), P)
  (bit P - 1 - i); the kept set is the recent window [P - recent, P) plus the
  ``heavy`` earlier tokens with the highest counts, the newer first on equal
  counts;
* decode at position t: the query attends the kept tokens plus t, every
  history shifts by one and takes the step's bit, token t starts with its own
  bit; if more than heavy + recent tokens remain, the lowest count among the
  tokens not in the recent window (t - recent, t] leaves, the oldest first on
  equal counts -- "keeps pivotal tokens with a higher probability" read as a
  deterministic rule.

The same loop as the H2O oracle with the accumulated score replaced by the
count.  Each bit also carries an ambiguity flag: set when the weight lies
within a relative band of the threshold, where float32 arithmetic on the GPU
may legitimately decide either way.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .attention import attend, causal_attention, causal_weights
from .h2o import prefill_select

MAX_WINDOW = 64
PIVOT_BAND = 1e-5       # relative half-width of the ambiguous zone around 1 / |A|


def window_mask(window: int) -> int:
    if not 1 <= window <= MAX_WINDOW:
        raise ValueError(f"window {window} outside [1, {MAX_WINDOW}]")
    return (1 << window) - 1


def pivotal(p: np.ndarray, n: int):
    """(bits, ambiguous): p >= 1 / n, and whether p is within the band of 1 / n."""
    thr = 1.0 / n
    p = np.asarray(p, dtype=np.float64)
    return p >= thr, np.abs(p - thr) <= PIVOT_BAND * thr


def count(h) -> np.ndarray:
    """Persistence count: set bits of each 64-bit history."""
    return np.bitwise_count(np.asarray(h, dtype=np.uint64)).astype(np.int64)


def prefill_histories(Q: np.ndarray, K: np.ndarray, scale: float, window: int):
    """(hist, amb) [P] uint64 for every prompt token.

    Row i of the causal softmax attends keys 0..i (i + 1 of them); key j gets
    bit P - 1 - i from each row i in [max(j, P - window), P).
    """
    P = Q.shape[0]
    p = causal_weights(Q, K, scale)
    hist = np.zeros(P, dtype=np.uint64)
    amb = np.zeros(P, dtype=np.uint64)
    for i in range(max(0, P - window), P):
        bits, near = pivotal(p[i, : i + 1], i + 1)
        b = np.uint64(1) << np.uint64(P - 1 - i)
        hist[: i + 1] |= np.where(bits, b, np.uint64(0))
        amb[: i + 1] |= np.where(near, b, np.uint64(0))
    return hist, amb


@dataclass
class Cache:
    """Kept positions with their histories and ambiguity masks (aligned arrays)."""
    pos: np.ndarray                      # int64
    hist: np.ndarray                     # uint64
    amb: np.ndarray                      # uint64


def prefill(Q: np.ndarray, K: np.ndarray, heavy: int, recent: int, window: int, scale: float):
    """Returns (cache, hist, amb) with hist/amb over the whole prompt."""
    hist, amb = prefill_histories(Q, K, scale, window)
    kept = prefill_select(count(hist).astype(np.float64), heavy, recent)
    return Cache(kept, hist[kept].copy(), amb[kept].copy()), hist, amb


def attend_step(cache: Cache, t: int, q: np.ndarray, K_all: np.ndarray, V_all: np.ndarray,
                scale: float, window: int, Kc: Optional[np.ndarray] = None, Vc: Optional[np.ndarray] = None):
    """Attention of the step-t query over the kept tokens plus t; every history
    shifts and takes this step's bit.  Returns (out, A, hist_A, amb_A, p).
    Kept tokens read Kc / Vc (cache slot contents), token t its own input."""
    A = np.append(cache.pos, t).astype(np.int64)
    Kc = K_all if Kc is None else Kc
    Vc = V_all if Vc is None else Vc
    p, out = attend(q, np.vstack([Kc[cache.pos], K_all[t:t + 1]]), np.vstack([Vc[cache.pos], V_all[t:t + 1]]), scale)
    bits, near = pivotal(p, len(A))
    wm = np.uint64(window_mask(window))
    one = np.uint64(1)
    h = (np.append(cache.hist, np.uint64(0)) << one | bits.astype(np.uint64)) & wm
    a = (np.append(cache.amb, np.uint64(0)) << one | near.astype(np.uint64)) & wm
    return out, A, h, a, p


def candidates(A: np.ndarray, t: int, recent: int) -> np.ndarray:
    """Indices into A of the positions outside the recent window (t - recent, t]."""
    return np.flatnonzero(A <= t - recent)


def victim(A: np.ndarray, hist_A: np.ndarray, t: int, recent: int) -> int:
    """Index into A of the token to evict: lowest count, then oldest position."""
    cand = candidates(A, t, recent)
    c = count(hist_A)
    return int(min(cand, key=lambda i: (c[i], A[i])))


def remove(A, hist_A, amb_A, idx: Optional[int]) -> Cache:
    if idx is None:
        return Cache(A, hist_A, amb_A)
    keep = np.ones(len(A), dtype=bool)
    keep[idx] = False
    return Cache(A[keep], hist_A[keep], amb_A[keep])


@dataclass
class Trajectory:
    prefill_kept: np.ndarray
    prefill_hist: np.ndarray             # histories of prefill_kept
    prompt_hist: np.ndarray              # histories of every prompt token
    out: np.ndarray                      # [T, d]
    evicted: np.ndarray                  # [T] position or -1
    final: Cache
    prompt_out: Optional[np.ndarray] = None
    steps: List[tuple] = field(default_factory=list)   # (A, p) per decode step, if recorded


def run_unit(Q_all: np.ndarray, K_all: np.ndarray, V_all: np.ndarray, P: int, heavy: int, recent: int,
             window: int, scale: float, steps: Optional[int] = None, want_prompt_out: bool = False,
             record: bool = False, Kc: Optional[np.ndarray] = None, Vc: Optional[np.ndarray] = None) -> Trajectory:
    """Prefill on the first P positions, then decode positions P..P+steps-1."""
    N = Q_all.shape[0]
    T = N - P if steps is None else steps
    budget = heavy + recent
    cache, hist, _ = prefill(Q_all[:P], K_all[:P], heavy, recent, window, scale)
    kept0, h0 = cache.pos.copy(), cache.hist.copy()
    prompt_out = causal_attention(Q_all[:P], K_all[:P], V_all[:P], scale)[1] if want_prompt_out else None
    outs, ev, rec = [], [], []
    for t in range(P, P + T):
        o, A, h, a, p = attend_step(cache, t, Q_all[t], K_all, V_all, scale, window, Kc, Vc)
        outs.append(o)
        if record:
            rec.append((A.copy(), p.copy()))
        if len(A) > budget:
            i = victim(A, h, t, recent)
            ev.append(int(A[i]))
            cache = remove(A, h, a, i)
        else:
            ev.append(-1)
            cache = Cache(A, h, a)
    d = V_all.shape[1]
    return Trajectory(kept0, h0, hist, np.array(outs).reshape(T, d), np.array(ev, dtype=np.int64),
                      cache, prompt_out, rec)
