"""Storage roundings used by the oracle (test infrastructure).

The method fixes no precision (the pages state none).  The oracle computes in
float64 and rounds only where a value is stored in the narrow type the
workload declares: RoPE'd q/k rows and the bf16 copy of h that a bf16
contraction consumes.  Each rounding is written from its definition:

* bf16: the nearest number with 8 significant bits (1 implicit + 7 stored),
  ties to the one whose last significant bit is even.  Normal range only; the
  workloads never produce values near bf16 under/overflow, and a value outside
  the normal range raises.
* fp32: IEEE binary32 round-to-nearest-even (NumPy's float64 -> float32 cast).
"""

from __future__ import annotations

import numpy as np

_BF16_SIG_BITS = 8
_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    Write |x| = m * 2**e with m in [0.5, 1).  A bf16 number has 8 significant
    bits, so the representable neighbours are multiples of 2**(e-8); scale by
    2**8, round half to even with rint, and scale back.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(m, _BF16_SIG_BITS)), e - _BF16_SIG_BITS)
    ax = np.abs(x)
    bad = (ax != 0) & ((ax < _BF16_MIN_NORMAL) | (np.abs(r) > _BF16_MAX))
    if np.any(bad) or not np.all(np.isfinite(x)):
        raise ValueError("value outside the bf16 normal range")
    return r


def round_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 values to IEEE fp32 (nearest even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_storage(x: np.ndarray, precision: str) -> np.ndarray:
    if precision == "bf16":
        return round_bf16(x)
    if precision == "fp32":
        return round_f32(x)
    if precision == "none":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(precision)


def table_values(arr: np.ndarray) -> np.ndarray:
    """Exact float64 values of a table stored as bf16 bits (uint16) or fp32."""
    a = np.asarray(arr)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.float64:
        return a
    raise TypeError(a.dtype)
