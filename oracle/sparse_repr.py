"""Sparse representation of a partially masked sequence (test infrastructure).

Page 1, key design 1 (and page 3, section 3.1 / Figure 4): a partially masked
sequence is represented by its clean tokens, the positions they occupy and the
total length.  The masked positions are exactly the positions no clean token
occupies, so the dense sequence is recovered without loss.  Page 1's example:
a 7-token sequence with clean tokens at positions 1, 2 and 4 (1-indexed) and
masks at 3, 5, 6, 7.

Positions here are 0-indexed; the register tokens that follow the sequence sit
at positions length .. length+R-1 (page 1, key design 2: consecutive ids right
after the sequence end).
"""

from __future__ import annotations

import numpy as np


def to_sparse(seq: np.ndarray, mask_id: int):
    """Dense sequence -> (clean tokens, their positions, total length)."""
    seq = np.asarray(seq)
    pos = np.nonzero(seq != mask_id)[0].astype(np.int64)
    return seq[pos].copy(), pos, int(seq.shape[0])


def from_sparse(tokens: np.ndarray, positions: np.ndarray, length: int, mask_id: int) -> np.ndarray:
    """(clean tokens, positions, length) -> dense sequence with mask_id elsewhere."""
    tokens = np.asarray(tokens)
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size and (positions.min() < 0 or positions.max() >= length):
        raise ValueError("position outside the sequence")
    if np.unique(positions).size != positions.size:
        raise ValueError("two clean tokens at one position")
    seq = np.full(length, mask_id, dtype=np.int64)
    seq[positions] = tokens
    return seq


def masked_positions(positions: np.ndarray, length: int) -> np.ndarray:
    """Positions not occupied by a clean token."""
    occ = np.zeros(length, dtype=bool)
    occ[np.asarray(positions, dtype=np.int64)] = True
    return np.nonzero(~occ)[0]


def register_positions(length: int, n_registers: int) -> np.ndarray:
    """Registers take consecutive position ids right after the sequence end."""
    return np.arange(length, length + n_registers, dtype=np.int64)
