"""Seeded inputs for the training-form (block-mask) attention.

A training sequence (page 1, key design 3; page 3, section 3.3) is the prompt
(block 0), the clean target tokens spread over blocks 1..M and the masked
target tokens over blocks M+1..M+N, each masked block followed by its own R
registers under the same block id.  Recipe (``SeedSequence([2026, index])``):

* a fraction ``mask_ratio`` of the generated tokens is masked; the clean and
  the masked tokens are cut into M and N non-empty blocks at random cut
  points (so block boundaries fall anywhere inside the 64-key tiles);
* rows are laid out in block order (prompt, clean blocks, then each masked
  block with its registers), or in a seeded random order when
  ``shuffle_rows`` is set (block ids are labels, not runs);
* q [B][n][H][d], k and v [B][n][H_kv][d]: N(0, 1) in fp32 rounded to bf16,
  standing for RoPE'd projections of unit-variance activations.

No attention arithmetic lives here.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from .generate import SEED_ROOT, bf16_bits_from_f32


@dataclass(frozen=True)
class TrainAttnConfig:
    name: str
    index: int
    batch: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    prompt_len: int
    gen_len: int
    n_registers: int
    clean_blocks: int          # M
    masked_blocks: int         # N
    mask_ratio: float = 0.5
    shuffle_rows: bool = False
    description: str = ""

    @property
    def n_masked(self) -> int:
        return int(round(self.gen_len * self.mask_ratio))

    @property
    def n_clean(self) -> int:
        return self.gen_len - self.n_masked

    @property
    def n_rows(self) -> int:
        return self.prompt_len + self.gen_len + self.masked_blocks * self.n_registers

    def replace(self, **kw) -> "TrainAttnConfig":
        return replace(self, **kw)


TRAIN_CONFIGS = [
    TrainAttnConfig(
        name="train_t2i_4k", index=20, batch=2, n_heads=32, n_kv_heads=32, head_dim=128,
        prompt_len=256, gen_len=4096, n_registers=64, clean_blocks=4, masked_blocks=4,
        description="4096-token T2I training sequence: 256 prompt, half of the image clean in 4 blocks, "
                    "half masked in 4 blocks with 64 registers each"),
    TrainAttnConfig(
        name="train_text", index=21, batch=4, n_heads=32, n_kv_heads=8, head_dim=128,
        prompt_len=512, gen_len=1024, n_registers=64, clean_blocks=8, masked_blocks=8,
        description="text training sequence: 512 prompt, 1024 generated (half clean in 8 blocks, "
                    "half masked in 8 blocks with 64 registers each), grouped heads 32/8"),
]


def get_train_config(name: str) -> TrainAttnConfig:
    for c in TRAIN_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def _cut(total: int, parts: int, rng: np.random.Generator) -> np.ndarray:
    """Sizes of `parts` non-empty pieces of `total` at random cut points."""
    if parts == 0 and total == 0:
        return np.empty(0, np.int64)
    if parts < 1 or parts > total:
        raise ValueError("cannot cut into that many non-empty blocks")
    cuts = np.sort(rng.choice(np.arange(1, total), parts - 1, replace=False)) if parts > 1 else np.empty(0, int)
    return np.diff(np.concatenate([[0], cuts, [total]])).astype(np.int64)


def block_layout(cfg: TrainAttnConfig, rng: np.random.Generator) -> np.ndarray:
    """Block id of every row of one sequence (int32 [n_rows])."""
    ids = [np.zeros(cfg.prompt_len, np.int64)]
    for j, size in enumerate(_cut(cfg.n_clean, cfg.clean_blocks, rng), start=1):
        ids.append(np.full(size, j))
    for j, size in enumerate(_cut(cfg.n_masked, cfg.masked_blocks, rng), start=cfg.clean_blocks + 1):
        ids.append(np.full(size + cfg.n_registers, j))
    blk = np.concatenate(ids)
    if cfg.shuffle_rows:
        blk = blk[rng.permutation(blk.size)]
    return blk.astype(np.int32)


@dataclass
class TrainAttnInputs:
    cfg: TrainAttnConfig
    q: np.ndarray            # uint16 bf16 bits [B][n][H][d]
    k: np.ndarray            # [B][n][H_kv][d]
    v: np.ndarray
    blocks: np.ndarray       # int32 [B][n]
    n_clean: np.ndarray      # int32 [B] (= M for every sequence)


def make_train_attn_inputs(cfg: TrainAttnConfig) -> TrainAttnInputs:
    ss = np.random.SeedSequence([SEED_ROOT, cfg.index])
    r_layout, r_q, r_k, r_v = (np.random.default_rng(s) for s in ss.spawn(4))
    n, B, d = cfg.n_rows, cfg.batch, cfg.head_dim

    def draw(rng, heads):
        x = rng.standard_normal((B, n, heads, d), dtype=np.float32)
        return bf16_bits_from_f32(x).reshape(B, n, heads, d)

    blocks = np.stack([block_layout(cfg, r_layout) for _ in range(B)])
    return TrainAttnInputs(cfg=cfg, q=draw(r_q, cfg.n_heads), k=draw(r_k, cfg.n_kv_heads),
                           v=draw(r_v, cfg.n_kv_heads), blocks=blocks,
                           n_clean=np.full(B, cfg.clean_blocks, dtype=np.int32))
