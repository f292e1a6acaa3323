"""Softmax attention in float64 (textbook definition).

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np


def softmax(x: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, with the maximum subtracted first.

    Entries equal to -inf get weight 0.
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def causal_weights(Q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Causal softmax weights of a prompt, p [P, P].

    p[i, j] = exp(scale q_i.k_j) / sum_{j' <= i} exp(scale q_i.k_j') for j <= i,
    and 0 above the diagonal: the query at position i sees keys 0..i, its own
    included.
    """
    P = Q.shape[0]
    s = (Q @ K.T) * scale
    s[np.triu_indices(P, 1)] = -np.inf
    return softmax(s)


def causal_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Causal self-attention of a prompt: returns (p [P, P], out = p V [P, d])."""
    p = causal_weights(Q, K, scale)
    return p, p @ V


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """One query over a set of keys/values: returns (p [n], out [d])."""
    p = softmax((K @ q) * scale)
    return p, p @ V
