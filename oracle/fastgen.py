"""FastGen per-head cache policies, in float64.

Test infrastructure only (see the package docstring).

[FG] Abstract and "提案手法" (proposed method): each attention head gets its own
cache policy -- drop long-range context on heads that attend locally, keep only
special tokens (and, per the policy list, punctuation) on heads centred on
them, keep the standard full cache on heads that attend broadly, and prune by
frequency (accumulated attention, the fixed "Frequency" cache of Figure 2's
caption, which cites H2O) -- with hybrids formed as unions ("Frequency+Local").

Readings (listed in the design notes): the local window W keeps positions
(t - W, t] after step t, so the step-t query sees [t - W, t]; the special
policy keeps exactly the prompt and decode positions whose token id is in the
keep set, and the step-t query also sees token t itself; frequency+local is
H2O with heavy = freq_heavy and recent = W; the full cache never evicts.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from . import h2o
from .attention import attend, causal_attention

FULL, H2O, LOCAL, SPECIAL = 0, 1, 2, 3


@dataclass
class Trajectory:
    prefill_kept: np.ndarray
    out: np.ndarray                      # [T, d]
    evicted: np.ndarray                  # [T] position leaving the cache at that step, or -1
    final_kept: np.ndarray
    prompt_out: Optional[np.ndarray] = None
    h2o: Optional[h2o.Trajectory] = None  # the full H2O record for FREQ+LOCAL heads


def run_full(Q_all, K_all, V_all, P, scale, steps=None, want_prompt_out=False) -> Trajectory:
    """Full cache: step t attends over every position 0..t; nothing is evicted."""
    T = Q_all.shape[0] - P if steps is None else steps
    outs = [attend(Q_all[t], K_all[:t + 1], V_all[:t + 1], scale)[1] for t in range(P, P + T)]
    po = causal_attention(Q_all[:P], K_all[:P], V_all[:P], scale)[1] if want_prompt_out else None
    return Trajectory(np.arange(P), np.array(outs).reshape(T, V_all.shape[1]), np.full(T, -1),
                      np.arange(P + T), po)


def run_local(Q_all, K_all, V_all, P, W, scale, steps=None, want_prompt_out=False) -> Trajectory:
    """Local window of W tokens: after step t the cache holds (t - W, t].

    The step-t query attends over [max(0, t - W), t]; position t - W leaves
    the cache at that step when t >= W.
    """
    T = Q_all.shape[0] - P if steps is None else steps
    outs, ev = [], []
    for t in range(P, P + T):
        lo = max(0, t - W)
        outs.append(attend(Q_all[t], K_all[lo:t + 1], V_all[lo:t + 1], scale)[1])
        ev.append(t - W if t >= W else -1)
    po = causal_attention(Q_all[:P], K_all[:P], V_all[:P], scale)[1] if want_prompt_out else None
    end = P + T
    return Trajectory(np.arange(max(0, P - W), P), np.array(outs).reshape(T, V_all.shape[1]),
                      np.array(ev), np.arange(max(0, end - W), end), po)


def run_special(Q_all, K_all, V_all, ids, keep_ids: Sequence[int], P, scale, steps=None,
                want_prompt_out=False) -> Trajectory:
    """Special + punctuation tokens only.

    The cache holds the positions whose id is in ``keep_ids``; the step-t query
    attends over those before t plus t itself, and t stays only if its id is
    in the keep set (otherwise it leaves at once and is logged as evicted).
    """
    T = Q_all.shape[0] - P if steps is None else steps
    keep = set(int(i) for i in keep_ids)
    kept = [j for j in range(P) if int(ids[j]) in keep]
    kept0 = np.array(kept, dtype=np.int64)
    outs, ev = [], []
    for t in range(P, P + T):
        A = np.array(kept + [t], dtype=np.int64)
        outs.append(attend(Q_all[t], K_all[A], V_all[A], scale)[1])
        if int(ids[t]) in keep:
            kept.append(t); ev.append(-1)
        else:
            ev.append(t)
    po = causal_attention(Q_all[:P], K_all[:P], V_all[:P], scale)[1] if want_prompt_out else None
    return Trajectory(kept0, np.array(outs).reshape(T, V_all.shape[1]), np.array(ev),
                      np.array(kept, dtype=np.int64), po)


def run_freq_local(Q_all, K_all, V_all, P, freq_heavy, W, scale, steps=None,
                   want_prompt_out=False) -> Trajectory:
    """Frequency + local hybrid: H2O with heavy = freq_heavy and recent = W."""
    tr = h2o.run_unit(Q_all, K_all, V_all, P, freq_heavy, W, scale, steps, want_prompt_out)
    return Trajectory(tr.prefill_kept, tr.out, tr.evicted, np.sort(tr.final.pos), tr.prompt_out, tr)


def run_unit(policy: int, Q_all, K_all, V_all, P, scale, *, heavy=0, recent=0, ids=None,
             keep_ids=(), steps=None, want_prompt_out=False) -> Trajectory:
    """Dispatch on the head's policy code (FULL=0, H2O=1, LOCAL=2, SPECIAL=3)."""
    if policy == FULL:
        return run_full(Q_all, K_all, V_all, P, scale, steps, want_prompt_out)
    if policy == LOCAL:
        return run_local(Q_all, K_all, V_all, P, recent, scale, steps, want_prompt_out)
    if policy == SPECIAL:
        return run_special(Q_all, K_all, V_all, ids, keep_ids, P, scale, steps, want_prompt_out)
    if policy == H2O:
        return run_freq_local(Q_all, K_all, V_all, P, heavy, recent, scale, steps, want_prompt_out)
    raise ValueError(policy)
