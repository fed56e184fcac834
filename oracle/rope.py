"""Rotary position embedding at explicit sparse position ids (test infrastructure).

The pages say clean tokens are encoded "with their position encoding" and the
masked positions are whatever the clean tokens do not occupy (page 1, key
design 1; page 3, section 3.1).  They name no encoding; this build reads it as
RoPE (rotary embedding) applied to each query/key row at its own position id,
so a sparse subset of positions is embedded exactly as it would be inside the
full sequence.

Convention (a reading; the pages fix none):

* pairs are interleaved: dims (2i, 2i+1), i = 0 .. d/2-1;
* frequency theta_i = base ** (-2i/d), evaluated in float64 with the C
  library's pow (``math.pow``);
* the table holds cos(pos*theta_i) and sin(pos*theta_i), evaluated in float64
  with the C library's cos/sin and rounded to fp32;
* the rotation (x0*c - x1*s, x0*s + x1*c) is evaluated in float64: each
  product of a bf16 or fp32 input with an fp32 table entry is exact in
  float64, so only the final sum rounds; the caller then rounds to storage.
"""

from __future__ import annotations

import math

import numpy as np


def frequencies(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base**(-2i/d) for i < d/2, float64."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    return np.array([math.pow(base, -2.0 * i / head_dim) for i in range(head_dim // 2)],
                    dtype=np.float64)


def table(max_pos: int, head_dim: int, base: float = 10000.0):
    """(cos, sin) tables [max_pos][d/2], computed in float64 and rounded to fp32."""
    theta = frequencies(head_dim, base)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rotate(x: np.ndarray, pos: np.ndarray, cos_t: np.ndarray, sin_t: np.ndarray) -> np.ndarray:
    """Rotate rows of x [..., n, d] (float64 holding bf16/fp32 values) by the
    angle of each row's position pos [..., n].  Returns float64 (unrounded)."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos)
    c = cos_t[pos].astype(np.float64)      # [..., n, d/2]
    s = sin_t[pos].astype(np.float64)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    # broadcast the per-row angle over any head axis between n and d
    while c.ndim < x0.ndim:
        c = c[..., None, :]
        s = s[..., None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out
