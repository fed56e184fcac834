"""From-scratch forward under the training-form block mask (test infrastructure).

Page 1, key design 3 (page 3, sections 3.3 and 7.3): training simulates the
incremental cache in one parallel forward.  The prompt is block 0, the clean
tokens are spread over blocks 1..M and the masked tokens over blocks
M+1..M+N; each masked block has its own copy of the registers with its block
id.  One forward then yields the outputs of several decode paths at once, e.g.
0->1->2->3->4 and 0->1->2->3->5.

This module materialises such a sequence for a given decode history and runs
every row through the same layers as the incremental loop, with visibility
from ``masks.block_mask``.  Cached incremental steps must reproduce its rows.
"""

from __future__ import annotations

import numpy as np

from .attention import attend
from .masks import block_mask
from .step import Model


def build_rows(model: Model, prompt_ids, clean_groups, masked_groups, prompt_pos=None):
    """Rows of the dense training-form sequence.

    clean_groups:  [(tokens, positions)] for blocks 1..M (decode history)
    masked_groups: [positions] for blocks M+1..M+N; each block is followed by
                   its own copy of the R registers.
    Returns ids, positions, block ids and, per masked block, the row indices
    of its masked tokens and of its registers.  The prompt sits at positions
    0 .. P-1 unless `prompt_pos` gives them (text infilling).
    """
    ids, pos, blk = [], [], []
    p = len(prompt_ids)
    ids += list(prompt_ids)
    pos += list(range(p)) if prompt_pos is None else [int(x) for x in prompt_pos]
    blk += [0] * p
    for j, (tok, ps) in enumerate(clean_groups, start=1):
        ids += list(tok)
        pos += list(ps)
        blk += [j] * len(tok)
    m = len(clean_groups)
    spans = []
    for j, ps in enumerate(masked_groups, start=m + 1):
        start = len(ids)
        ids += [model.mask_id] * len(ps)
        pos += list(ps)
        blk += [j] * len(ps)
        reg0 = len(ids)
        ids += list(model.register_ids())
        pos += list(model.register_pos())
        blk += [j] * model.n_registers
        spans.append((np.arange(start, reg0), np.arange(reg0, len(ids))))
    return (np.array(ids, np.int64), np.array(pos, np.int64), np.array(blk, np.int64), m, spans)


def dense_forward(model: Model, ids, pos, blocks, n_clean_blocks: int):
    """Every row through every layer under the block mask; per-layer outputs [n, hidden]."""
    vis = block_mask(blocks, blocks, n_clean_blocks)
    outs = []
    q, k, v = model.qkv_layer1(ids, pos)
    o = attend(q, k, v, vis).reshape(len(ids), model.hidden)
    outs.append(o)
    if model.layer2 is not None:
        q, k, v = model.qkv_layer2(o, pos)
        o = attend(q, k, v, vis).reshape(len(ids), model.hidden)
        outs.append(o)
    return outs
