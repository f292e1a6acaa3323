"""4-bit cached keys and values (the Scissorhands page's 4-bit combination).

Test infrastructure only (see the package docstring).

[SH] Abstract: the cache compression combines with 4-bit quantisation for a
further reduction.  The page names no format, so the format is a reading
(listed in the design notes): each cached key or value row is split into
groups of 32 consecutive elements; a group's scale is its largest magnitude
times the float32 value of 1/7, and each element's code is its float32
quotient by the scale rounded half to even and clamped to [-7, 7] (a zero
group has scale 0 and codes 0).  Scale, quotient and rounding are float32
operations, so both this oracle and the GPU take every integer decision in
the same precision.  A cached row reads back as code * scale.  Rows are
quantised when they enter the cache; the step-t query still uses token t's
own key and value at full precision at that step.
"""

from __future__ import annotations

import numpy as np

GROUP = 32
QMAX = 7
INV_QMAX = np.float32(1.0 / 7.0)


def quantize_rows(X: np.ndarray):
    """Rows X [n, d] (d a multiple of 32) -> (codes int8 [n, d], scales float32 [n, d / 32])."""
    X32 = np.asarray(X, dtype=np.float32)
    n, d = X32.shape
    if d % GROUP:
        raise ValueError("row length must be a multiple of 32")
    g = X32.reshape(n, d // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=-1)
    scale = (amax * INV_QMAX).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint((g / safe[..., None]).astype(np.float32))     # a zero group: 0 / 1 -> code 0
    codes = np.clip(q, -QMAX, QMAX).astype(np.int8).reshape(n, d)
    return codes, scale


def dequantize_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """code * scale per element, in float64 (exact: a 4-bit code times a float32)."""
    n, d = codes.shape
    g = codes.reshape(n, d // GROUP, GROUP).astype(np.float64) * scale.astype(np.float64)[..., None]
    return g.reshape(n, d)


def roundtrip(X: np.ndarray) -> np.ndarray:
    """What a 4-bit cache slot holding each row of X reads back."""
    return dequantize_rows(*quantize_rows(X))
