"""HashEvict: pre-attention eviction by Hamming distance of sign sketches.

Test infrastructure only (see the package docstring).

[HE] 要約 / original abstract: the cache keeps a small binary structure in GPU
memory -- sign-binarised Gaussian projections of the keys, with a projection
length far below the head dimension.  Each decode step compares the current
query's binarised projection with every cached key's by Hamming distance
(a proxy for cosine dissimilarity), and before any attention is computed the
new token's key and value replace the token expected to receive the least
attention: the one at the largest distance.

Readings (listed in the design notes):

* sketch(x) has bit b set iff the exact value of sum_i W[i, b] x[i] is > 0
  (a zero sum gives 0); bit b is the b-th least significant bit;
* ties in distance evict the oldest position;
* no recent window; the new token is always inserted, and the step-t query
  attends over the cache after the replacement (t included);
* the prompt is replayed through the same rule: the cache starts as positions
  [0, B) and each later prompt position i replaces the farthest key from
  sketch(q_i) (no attention is needed for that).
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .attention import attend, causal_attention


def sketches(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Packed sign sketches of the rows of X [n, d] under W [d, bits] (bits <= 64).

    The sign is that of the exact dot product.  Entries are exact float64
    values (bf16 inputs: every product is exact).  A float64 dot of n terms
    differs from the exact value by at most gamma_n * sum|terms| with
    gamma_n = n u / (1 - n u), u = 2^-53, whatever the summation order.  The
    sum of magnitudes is itself computed in float64, so it may fall short of
    the exact one by a relative gamma_n, and the bound's product rounds once
    more; gamma_{2n+2} exceeds gamma_n / ((1 - gamma_n)(1 - u)), so the test
    below never misses a fragile dot.  A dot inside that bound is recomputed
    with math.fsum (correctly rounded, so its sign is exact).
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    n, d = X.shape
    bits = W.shape[1]
    s = X @ W
    u = 2.0 ** -53
    m = 2 * d + 2
    gamma = m * u / (1.0 - m * u)
    bound = gamma * (np.abs(X) @ np.abs(W))
    fragile = np.argwhere(np.abs(s) <= bound)
    for i, b in fragile:
        s[i, b] = math.fsum((X[i] * W[:, b]).tolist())
    out = np.zeros(n, dtype=np.uint64)
    for b in range(bits):
        out |= (s[:, b] > 0).astype(np.uint64) << np.uint64(b)
    return out


def hamming(a, b) -> np.ndarray:
    """Number of differing bits between packed sketches (population count of a XOR b)."""
    return np.bitwise_count(np.bitwise_xor(np.asarray(a, dtype=np.uint64),
                                           np.asarray(b, dtype=np.uint64))).astype(np.int64)


def farthest(qsk: int, cache_pos: np.ndarray, ksk: np.ndarray) -> int:
    """Index into cache_pos of the key farthest from qsk: largest distance, then oldest."""
    h = hamming(np.uint64(qsk), ksk[cache_pos])
    at_max = np.flatnonzero(h == h.max())
    return int(at_max[np.argmin(cache_pos[at_max])])


def replay_prompt(qsk: np.ndarray, ksk: np.ndarray, P: int, B: int) -> np.ndarray:
    """Cache after the prompt: positions [0, min(P, B)), then for i = B..P-1 the
    farthest key from sketch(q_i) is replaced by i."""
    cache = np.arange(min(P, B), dtype=np.int64)
    for i in range(B, P):
        v = farthest(int(qsk[i]), cache, ksk)
        cache[v] = i
    return cache


@dataclass
class Trajectory:
    prefill_kept: np.ndarray             # sorted
    out: np.ndarray                      # [T, d]
    evicted: np.ndarray                  # [T]
    final_kept: np.ndarray               # sorted
    qsk: np.ndarray
    ksk: np.ndarray
    prompt_out: Optional[np.ndarray] = None


def run_unit(Q_all, K_all, V_all, W, P, B, scale, steps=None, want_prompt_out=False,
             qsk=None, ksk=None, Kc=None, Vc=None) -> Trajectory:
    """Prompt replay, then decode positions P..P+steps-1 with pre-attention replacement.

    Kc / Vc: what a cache slot holding each position reads back (lossy cache
    formats; the full sequences otherwise).  Sketches are taken from the
    inputs when a token enters; the step attends the cache after the
    replacement, so token t is read from its slot like every kept token.
    """
    Kc = K_all if Kc is None else Kc
    Vc = V_all if Vc is None else Vc
    N = Q_all.shape[0]
    T = N - P if steps is None else steps
    if qsk is None:
        qsk = sketches(Q_all[:P + T], W)
    if ksk is None:
        ksk = sketches(K_all[:P + T], W)
    cache = replay_prompt(qsk, ksk, P, B)
    kept0 = np.sort(cache)
    cache = list(cache)
    outs, ev = [], []
    for t in range(P, P + T):
        if len(cache) >= B:
            v = farthest(int(qsk[t]), np.array(cache, dtype=np.int64), ksk)
            ev.append(int(cache[v]))
            cache[v] = t
        else:
            ev.append(-1)
            cache.append(t)
        A = np.array(cache, dtype=np.int64)
        outs.append(attend(Q_all[t], Kc[A], Vc[A], scale)[1])
    po = causal_attention(Q_all[:P], K_all[:P], V_all[:P], scale)[1] if want_prompt_out else None
    return Trajectory(kept0, np.array(outs).reshape(T, V_all.shape[1]), np.array(ev, dtype=np.int64),
                      np.sort(np.array(cache, dtype=np.int64)), qsk, ksk, po)
