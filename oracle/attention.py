"""Masked multi-head attention in float64 (test infrastructure).

softmax(q k^T / sqrt(d)) v over the keys a query row may see, per head.  With
grouped-query attention (H query heads, H_kv key/value heads) query head h uses
key/value head floor(h / (H / H_kv)) (a reading; the pages use plain
multi-head attention).  Which keys a row may see comes from ``masks``.
"""

from __future__ import annotations

import math

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """q [n_q, H, d], k/v [n_k, H_kv, d], visible bool [n_q, n_k] -> O [n_q, H, d]."""
    n_q, n_h, d = q.shape
    n_k, n_kv, _ = k.shape
    if n_h % n_kv:
        raise ValueError("H must be a multiple of H_kv")
    if visible.shape != (n_q, n_k):
        raise ValueError("visibility shape")
    if n_q and not np.all(visible.any(axis=1)):
        raise ValueError("a query row sees no key")
    g = n_h // n_kv
    qh = q.transpose(1, 0, 2).reshape(n_kv, g * n_q, d)
    kh = k.transpose(1, 0, 2)
    vh = v.transpose(1, 0, 2)
    s = (qh @ kh.transpose(0, 2, 1)) / math.sqrt(d)
    vis = np.tile(visible, (g, 1))[None]
    s = np.where(vis, s, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    o = (p @ vh) / p.sum(axis=-1, keepdims=True)
    return o.reshape(n_h, n_q, d).transpose(1, 0, 2)


def attend_bruteforce(q, k, v, visible) -> np.ndarray:
    """The same quantity written element by element (tiny inputs only)."""
    n_q, n_h, d = q.shape
    n_k, n_kv, _ = k.shape
    g = n_h // n_kv
    out = np.zeros((n_q, n_h, d))
    for h in range(n_h):
        kvh = h // g
        for i in range(n_q):
            keys = [j for j in range(n_k) if visible[i, j]]
            scores = [sum(float(q[i, h, t]) * float(k[j, kvh, t]) for t in range(d)) / math.sqrt(d)
                      for j in keys]
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for t in range(d):
                out[i, h, t] = sum(wj * float(v[j, kvh, t]) for wj, j in zip(w, keys)) / tot
    return out
