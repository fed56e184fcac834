"""Seeded synthetic inputs: folded q/k/v tables, the vocab head, prompt ids,
per-step decode counts and the pre-generated unmask order.

Recipe (all streams from ``numpy.random.SeedSequence([2026, cfg.index])``):

* fp32 workload (tiny case): an embedding E[V+1+R][hidden] and projections
  Wq/Wk/Wv[hidden][heads*d], all i.i.d. normal with variance 1/sqrt(hidden);
  the folded tables Tq = E Wq (etc.) are formed in float64 and rounded to fp32.
  The vocab head W[V][hidden] uses the same distribution.
* bf16 workloads: folded tables and the vocab head drawn directly as N(0, 1)
  in fp32 and rounded to bf16 (round to nearest even).  This stands for
  activations N(0,1) scaled by 1/sqrt(hidden) times unit-variance projections:
  the projected q/k/v rows are O(1) either way.
* prompt token ids uniform in [0, V).
* unmask order: a seeded permutation (random order), or the 2D cell
  round-robin below (stratified order); semi-autoregressive text has no
  pre-generated order (confidence decides inside each block).

The per-step decode counts and the order are inputs the sampler is handed;
the hot path never draws random numbers.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .configs import Config

SEED_ROOT = 2026
_CHUNK_ROWS = 4096


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> the exact fp32 value."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def cosine_counts(gen_len: int, n_steps: int) -> np.ndarray:
    """Tokens decoded per step under the cosine schedule.

    M_k = floor(L cos(pi/2 * k/K)) masked tokens remain after step k
    (M_0 = L, M_K = 0); step k decodes n_k = M_{k-1} - M_k tokens.
    """
    m = [gen_len] + [math.floor(gen_len * math.cos(math.pi / 2.0 * k / n_steps))
                     for k in range(1, n_steps)] + [0]
    n = np.array([m[k - 1] - m[k] for k in range(1, n_steps + 1)], dtype=np.int32)
    if n.sum() != gen_len or n.min() < 1:
        raise ValueError(f"cosine schedule degenerate for L={gen_len}, K={n_steps}")
    return n


def stratified_order_2d(grid: int, rng: np.random.Generator, cell: int = 4) -> np.ndarray:
    """Raster indices of a grid x grid image in a 2D-stratified random order.

    The grid is tiled into cell x cell squares.  Each square's positions are
    shuffled once; then for round j = 0 .. cell*cell-1 the squares are visited
    in a freshly shuffled order and each contributes its j-th position.  Every
    aligned run of (#squares) entries therefore covers each square once, so
    any prefix of the order is spread over the whole image.
    """
    if grid % cell:
        raise ValueError("grid must be a multiple of the cell size")
    cps = grid // cell
    n_cells = cps * cps
    members = np.empty((n_cells, cell * cell), dtype=np.int64)
    for c in range(n_cells):
        cy, cx = divmod(c, cps)
        ys = cy * cell + np.arange(cell)
        xs = cx * cell + np.arange(cell)
        idx = (ys[:, None] * grid + xs[None, :]).reshape(-1)
        members[c] = rng.permutation(idx)
    out = np.empty(grid * grid, dtype=np.int64)
    for j in range(cell * cell):
        perm = rng.permutation(n_cells)
        out[j * n_cells:(j + 1) * n_cells] = members[perm, j]
    return out


@dataclass
class SemiARStep:
    block: int          # block index (left to right)
    sub: int            # sub-step within the block
    n_cand: int         # still-masked positions of the block
    n_select: int       # positions unmasked at this sub-step


@dataclass
class Workload:
    cfg: Config
    tq: np.ndarray                   # [V+1+R][H*d]   uint16 bf16 bits | float32
    tk: np.ndarray                   # [V+1+R][Hkv*d]
    tv: np.ndarray                   # [V+1+R][Hkv*d]
    w_vocab: np.ndarray              # [V][hidden]
    prompt_ids: np.ndarray           # int32 [B][P]
    order: Optional[np.ndarray]      # int32 [B][L] absolute positions, or None
    counts: np.ndarray               # int32 [n_steps]: decode counts (C) per step
    semi_ar: list = field(default_factory=list)   # [SemiARStep] for semi-AR text
    prompt_pos: Optional[np.ndarray] = None       # int32 [B][P] positions of the prompt tokens
    gen_pos: Optional[np.ndarray] = None          # int32 [B][L] masked positions, ascending
    layer_w: list = field(default_factory=list)   # upper layers' projections [proj_rows][hidden] bf16

    def __post_init__(self):
        cfg = self.cfg
        if self.prompt_pos is None:
            self.prompt_pos = np.tile(np.arange(cfg.prompt_len, dtype=np.int32), (cfg.batch, 1))
        if self.gen_pos is None:
            self.gen_pos = np.tile(np.arange(cfg.prompt_len, cfg.seq_len, dtype=np.int32), (cfg.batch, 1))

    @property
    def is_bf16(self) -> bool:
        return self.cfg.precision == "bf16"


def _seed_streams(cfg: Config):
    ss = np.random.SeedSequence([SEED_ROOT, cfg.index])
    kids = ss.spawn(9)      # later streams (text variants, upper layers) leave the first ones unchanged
    return [np.random.default_rng(k) for k in kids]


def infill_positions(seq_len: int, gen_len: int, n_spans: int, rng: np.random.Generator):
    """(clean, masked) positions: `gen_len` masked positions in `n_spans`
    non-empty spans placed at random inside [0, seq_len), with at least one
    clean position before every span."""
    n_clean = seq_len - gen_len
    if n_spans < 1 or n_spans > gen_len or n_spans > n_clean:
        raise ValueError("infill spans do not fit")
    cuts = np.sort(rng.choice(np.arange(1, gen_len), n_spans - 1, replace=False)) if n_spans > 1 else []
    lengths = np.diff(np.concatenate([[0], cuts, [gen_len]])).astype(np.int64)
    # clean tokens before each span (>= 1) and after the last one (>= 0)
    gaps = np.ones(n_spans + 1, dtype=np.int64)
    gaps[-1] = 0
    extra = n_clean - int(gaps.sum())
    gaps += np.bincount(rng.integers(0, n_spans + 1, size=extra), minlength=n_spans + 1)
    masked = np.zeros(seq_len, dtype=bool)
    at = 0
    for j in range(n_spans):
        at += int(gaps[j])
        masked[at:at + int(lengths[j])] = True
        at += int(lengths[j])
    pos = np.arange(seq_len, dtype=np.int32)
    return pos[~masked], pos[masked]


def _normal_bf16(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        out[r0:r1] = bf16_bits_from_f32(rng.standard_normal((r1 - r0, cols), dtype=np.float32))
    return out


def _counts(cfg: Config) -> np.ndarray:
    if cfg.schedule == "fixed":
        n = np.full(cfg.n_steps, cfg.per_step, dtype=np.int32)
        if n.sum() != cfg.gen_len:
            raise ValueError("fixed schedule does not cover the generated length")
        return n
    if cfg.schedule == "cosine":
        return cosine_counts(cfg.gen_len, cfg.n_steps)
    if cfg.schedule == "semi_ar":
        return np.array([s.n_cand for s in semi_ar_plan(cfg)], dtype=np.int32)
    raise ValueError(cfg.schedule)


def semi_ar_plan(cfg: Config, block_seq=None) -> list:
    """Blocks left to right (or in `block_seq` order); each block is unmasked
    over `steps_per_block` sub-steps of block/steps_per_block tokens each.
    Block j holds the generated positions [j*block, (j+1)*block) in position
    order."""
    if cfg.gen_len % cfg.block or cfg.block % cfg.steps_per_block:
        raise ValueError("block sizes do not divide")
    per = cfg.block // cfg.steps_per_block
    plan = []
    for b in (range(cfg.gen_len // cfg.block) if block_seq is None else block_seq):
        for s in range(cfg.steps_per_block):
            plan.append(SemiARStep(block=b, sub=s, n_cand=cfg.block - s * per, n_select=per))
    if len(plan) != cfg.n_steps:
        raise ValueError("semi-AR plan length differs from n_steps")
    return plan


def make_workload(cfg: Config, tables: bool = True) -> Workload:
    """Build the seeded synthetic workload of `cfg`.

    With tables=False the (large) tables are replaced by empty arrays; prompt
    ids, counts and orders are still drawn from their own streams, so they do
    not depend on this flag.
    """
    r_tq, r_tk, r_tv, r_w, r_prompt, r_order, r_emb, r_text, r_layers = _seed_streams(cfg)
    rows, hd, kvd = cfg.table_rows, cfg.hidden, cfg.n_kv_heads * cfg.head_dim
    if not tables:
        dt = np.uint16 if cfg.precision == "bf16" else np.float32
        tq = np.empty((0, hd), dt)
        tk = np.empty((0, kvd), dt)
        tv = np.empty((0, kvd), dt)
        w = np.empty((0, hd), dt)
    elif cfg.precision == "bf16":
        tq = _normal_bf16(r_tq, rows, hd)
        tk = _normal_bf16(r_tk, rows, kvd)
        tv = _normal_bf16(r_tv, rows, kvd)
        w = _normal_bf16(r_w, cfg.vocab, hd)
    elif cfg.precision == "fp32":
        std = 1.0 / math.sqrt(math.sqrt(hd))   # variance 1/sqrt(hidden)
        emb = r_emb.standard_normal((rows, hd)) * std
        wq = r_tq.standard_normal((hd, hd)) * std
        wk = r_tk.standard_normal((hd, kvd)) * std
        wv = r_tv.standard_normal((hd, kvd)) * std
        tq = (emb @ wq).astype(np.float32)
        tk = (emb @ wk).astype(np.float32)
        tv = (emb @ wv).astype(np.float32)
        w = (r_w.standard_normal((cfg.vocab, hd)) * std).astype(np.float32)
    else:
        raise ValueError(cfg.precision)

    # upper layers: W_l [proj_rows][hidden] bf16, rows = q heads | k heads | v heads,
    # N(0, 1) * 2 / sqrt(hidden): the head outputs of a layer are averages of
    # O(1) values over many keys (rms ~0.3), and this gain keeps each layer's
    # output at the first layer's scale (rms ratio 1.1-1.3 on the test shapes),
    # so the last layer's confidences are not saturated
    layer_w = []
    if cfg.layers > 1:
        if cfg.precision != "bf16":
            raise ValueError("upper layers are defined for bf16 workloads")
        for _ in range(cfg.layers - 1):
            if tables:
                x = r_layers.standard_normal((cfg.proj_rows, hd), dtype=np.float32) * np.float32(2.0 / math.sqrt(hd))
                layer_w.append(bf16_bits_from_f32(x))
            else:
                layer_w.append(np.empty((0, hd), np.uint16))

    prompt = r_prompt.integers(0, cfg.vocab, size=(cfg.batch, cfg.prompt_len)).astype(np.int32)

    order = None
    if cfg.order == "random":
        order = np.stack([r_order.permutation(cfg.gen_len) for _ in range(cfg.batch)])
    elif cfg.order == "stratified2d":
        if cfg.grid * cfg.grid != cfg.gen_len:
            raise ValueError("image grid does not match the generated length")
        order = np.stack([stratified_order_2d(cfg.grid, r_order) for _ in range(cfg.batch)])
    if order is not None:
        order = (order + cfg.prompt_len).astype(np.int32)

    block_seq = None
    if cfg.block_order == "random":
        if cfg.schedule != "semi_ar":
            raise ValueError("a block order needs the semi-AR schedule")
        block_seq = r_text.permutation(cfg.gen_len // cfg.block).tolist()
    elif cfg.block_order != "ltr":
        raise ValueError(cfg.block_order)
    prompt_pos = gen_pos = None
    if cfg.infill_spans:
        if order is not None:
            raise ValueError("infilling is defined for the semi-AR schedule")
        pairs = [infill_positions(cfg.seq_len, cfg.gen_len, cfg.infill_spans, r_text) for _ in range(cfg.batch)]
        prompt_pos = np.stack([c for c, _ in pairs]).astype(np.int32)
        gen_pos = np.stack([m for _, m in pairs]).astype(np.int32)
    plan = semi_ar_plan(cfg, block_seq) if cfg.schedule == "semi_ar" else []
    return Workload(cfg=cfg, tq=tq, tk=tk, tv=tv, w_vocab=w, prompt_ids=prompt,
                    order=order, counts=_counts(cfg), semi_ar=plan, prompt_pos=prompt_pos, gen_pos=gen_pos,
                    layer_w=layer_w)
