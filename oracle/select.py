"""Which positions are unmasked after a step (test infrastructure).

Page 3, section 3.2 (and page 1, worked example): for text-to-image and image
editing the unmasking order is generated in advance, with no confidence
scores, so every position decoded at a step is unmasked.  For text the blocks
go left to right and, within a block, confidence scores decide which tokens to
unmask.  Reading for the text case: the n highest-confidence positions of the
block are unmasked, ties broken towards the lower position; the others stay
masked for the next sub-step.
"""

from __future__ import annotations

import numpy as np


def select_all(cand_pos: np.ndarray):
    """Pre-generated order: every candidate is unmasked, in the given order."""
    cand_pos = np.asarray(cand_pos)
    return np.arange(cand_pos.size), np.empty(0, dtype=np.int64)


def select_by_confidence(cand_pos: np.ndarray, conf32: np.ndarray, n_select: int):
    """Indices (into the candidate list) of the unmasked and of the still-masked
    candidates, each listed in ascending position order."""
    cand_pos = np.asarray(cand_pos, dtype=np.int64)
    conf32 = np.asarray(conf32, dtype=np.float64)
    if not 0 <= n_select <= cand_pos.size:
        raise ValueError("n_select out of range")
    ranked = sorted(range(cand_pos.size), key=lambda i: (-conf32[i], cand_pos[i]))
    chosen = set(ranked[:n_select])
    by_pos = sorted(range(cand_pos.size), key=lambda i: cand_pos[i])
    sel = np.array([i for i in by_pos if i in chosen], dtype=np.int64)
    rem = np.array([i for i in by_pos if i not in chosen], dtype=np.int64)
    return sel, rem
