"""Step-causal attention masks (test infrastructure).

Inference form (page 1, worked example = paper Figure 3; page 3, Figure 3):
at step k the model sees four kinds of tokens - tokens already in the KV cache,
tokens decoded at step k-1 that enter the cache now ("new"), the masked tokens
decoded at step k ("decode") and the registers.  New tokens may not attend to
the current masked tokens or registers, so the cache is never polluted by them;
registers attend to everything and are attended to only by the current masked
tokens and registers.  Cached tokens are not queried.  The reading used here
for the remaining pairs: new tokens see the cache and each other; decode tokens
see everything present this step, registers included.

Training form (page 1, key design 3; page 3, sections 3.3 and 7.3; page 4,
method 2): the prompt is block 0, clean tokens are assigned to blocks 1..M and
masked tokens to blocks M+1..M+N (block ids are labels, not contiguous runs).
A clean (or prompt) block i attends to blocks j <= i.  A masked block i attends
to itself and to every block j <= M, but not to other masked blocks.  Each
masked block carries its own registers under the same block id.
"""

from __future__ import annotations

import numpy as np

CACHED, NEW, DECODE, REGISTER = "cached", "new", "decode", "register"

_SEES = {
    NEW: {CACHED, NEW},
    DECODE: {CACHED, NEW, DECODE, REGISTER},
    REGISTER: {CACHED, NEW, DECODE, REGISTER},
}


def kind_visible(query_kind: str, key_kind: str) -> bool:
    """May a query row of `query_kind` attend to a key of `key_kind`?"""
    if query_kind == CACHED:
        raise ValueError("cached tokens are not queried")
    return key_kind in _SEES[query_kind]


def inference_mask(query_kinds, key_kinds) -> np.ndarray:
    """Boolean [n_q, n_k] visibility from the inference rule."""
    return np.array([[kind_visible(q, k) for k in key_kinds] for q in query_kinds], dtype=bool)


def step_kinds(n_cache: int, n_new: int, n_decode: int, n_reg: int):
    """Kinds of the query rows [new | decode | register] and of the keys
    [cache | new | decode | register] of one sampling step."""
    q = [NEW] * n_new + [DECODE] * n_decode + [REGISTER] * n_reg
    k = [CACHED] * n_cache + [NEW] * n_new + [DECODE] * n_decode + [REGISTER] * n_reg
    return q, k


def step_mask(n_cache: int, n_new: int, n_decode: int, n_reg: int) -> np.ndarray:
    q, k = step_kinds(n_cache, n_new, n_decode, n_reg)
    return inference_mask(q, k)


def block_mask(q_blocks, k_blocks, n_clean_blocks: int) -> np.ndarray:
    """Training-form visibility from block ids; blocks 0..M are prompt/clean,
    blocks > M are masked (M = n_clean_blocks)."""
    qb = np.asarray(q_blocks)[:, None]
    kb = np.asarray(k_blocks)[None, :]
    m = n_clean_blocks
    clean_q = qb <= m
    return np.where(clean_q, kb <= qb, (kb == qb) | (kb <= m))
