"""Subset logits, confidence and argmax (test infrastructure).

Page 1, key design 1: the reverse process factorises over positions, so only
the positions being decoded need logits; a dense model would emit an L x V
logits tensor that is mostly unused.  Page 3, section 3.2: logits are produced
only for the tokens to decode.  The pages say "sample" and "confidence" without
a formula; the reading here is greedy decoding (argmax, lowest vocab index on
ties) and confidence = the largest softmax probability at temperature 1.

Where floating point decides an integer, the decision is taken in fp32, the
precision the HIP path decides in: the argmax runs over the fp32-rounded
logits, and confidences are compared as fp32 values.
"""

from __future__ import annotations

import numpy as np

from .numerics import round_f32


def subset_logits(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """z = h W^T for the decoded rows only: h [n, hidden], W [V, hidden] -> [n, V]."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def logsumexp(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]


def decide(z: np.ndarray):
    """Per row: (token, conf32, conf64, margin).

    token  = first index of the maximum of the fp32-rounded logits;
    conf64 = exp(max z - logsumexp z) = the largest softmax probability;
    conf32 = conf64 rounded to fp32 (the value confidence decisions compare);
    margin = largest minus second-largest logit (float64), a certificate of
             how far the argmax is from a tie.
    """
    z = np.asarray(z, dtype=np.float64)
    token = np.argmax(round_f32(z), axis=-1)
    conf64 = np.exp(z.max(axis=-1) - logsumexp(z))
    top2 = -np.sort(-z, axis=-1)[..., :2]
    margin = top2[..., 0] - top2[..., 1] if z.shape[-1] > 1 else np.full(z.shape[:-1], np.inf)
    return token.astype(np.int64), round_f32(conf64), conf64, margin


def top_two(z: np.ndarray):
    """Per row the two best (index, value) pairs of the float64 logits, in rank
    order: larger value first, lower index on equal values.  Returns idx [n, 2]
    (int64) and val [n, 2] (float64).  Used as the reference for the per-decision
    certificate (how far the decision is from a tie, and how close a measured
    logit is to the exact one)."""
    z = np.asarray(z, dtype=np.float64)
    # a stable sort of -z keeps equal values in index order
    order = np.argsort(-z, axis=-1, kind="stable")[..., :2]
    return order.astype(np.int64), np.take_along_axis(z, order, axis=-1)
