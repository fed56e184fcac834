"""The five workload configurations of the sparse sampling step.

Shapes follow the Sparse-LaViDa pages: 64 register tokens (page 1, key design
2; page 3, section 3.1), 1024x1024 images as 4096 tokens and 1024-token images
(page 1, motivation and key design 2), editing with a reference image in the
prompt (page 1, main results), text generation of length 1024 in blocks of 32
(page 3, section 4.4).  Head counts, vocabulary sizes and prompt lengths are
workload choices, not from the pages.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    index: int                 # seed stream index
    batch: int                 # B independent sequences
    n_heads: int               # H query heads
    n_kv_heads: int            # H_kv key/value heads (GQA when < H)
    head_dim: int              # d
    vocab: int                 # V; mask id = V, register ids V+1 .. V+R
    prompt_len: int            # P prompt tokens at positions 0 .. P-1
    gen_len: int               # L generated positions at P .. P+L-1
    n_registers: int           # R registers at positions P+L .. P+L+R-1
    n_steps: int               # sampling steps
    schedule: str              # "fixed" | "cosine" | "semi_ar"
    order: str                 # "random" | "stratified2d" | "confidence"
    precision: str             # "fp32" | "bf16"
    grid: int = 0              # image grid side for 2D orders
    per_step: int = 0          # fixed schedule: tokens per step
    block: int = 0             # semi-AR block size
    steps_per_block: int = 0   # semi-AR sub-steps per block
    block_order: str = "ltr"   # semi-AR: "ltr" (left to right) | "random" (seeded block order)
    infill_spans: int = 0      # > 0: the generated positions are this many masked spans
                               # placed inside the sequence (text infilling), the clean
                               # prompt tokens fill the other positions
    layers: int = 1            # attention layers; layer l > 1 projects the previous
                               # layer's head outputs with its own weights (bf16 only)
    rope_theta: float = 10000.0
    description: str = ""

    @property
    def hidden(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def seq_len(self) -> int:
        """Total length of the sequence (prompt + generated)."""
        return self.prompt_len + self.gen_len

    @property
    def table_rows(self) -> int:
        """Rows of the folded q/k/v tables: V tokens, the mask token, R registers."""
        return self.vocab + 1 + self.n_registers

    @property
    def mask_id(self) -> int:
        return self.vocab

    @property
    def proj_rows(self) -> int:
        """Output features of an upper layer's projection: q heads, k heads, v heads."""
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    @property
    def select_per_step(self) -> int:
        """Semi-AR: tokens unmasked per sub-step."""
        return self.block // self.steps_per_block if self.schedule == "semi_ar" else 0

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = (
    Config(
        name="c1_tiny", index=0, batch=1, n_heads=4, n_kv_heads=4, head_dim=64,
        vocab=512, prompt_len=16, gen_len=48, n_registers=8, n_steps=6,
        schedule="fixed", per_step=8, order="random", precision="fp32",
        description="tiny CPU-seconds case, fp32, 6 steps x 8 tokens, random order",
    ),
    Config(
        name="c2_t2i_1k", index=1, batch=1, n_heads=32, n_kv_heads=32, head_dim=128,
        vocab=8192, prompt_len=128, gen_len=1024, n_registers=64, n_steps=64,
        schedule="cosine", order="stratified2d", grid=32, precision="bf16",
        description="text-to-image, 32x32 image tokens + 128 text tokens",
    ),
    Config(
        name="c3_t2i_4k", index=2, batch=4, n_heads=32, n_kv_heads=32, head_dim=128,
        vocab=8192, prompt_len=256, gen_len=4096, n_registers=64, n_steps=64,
        schedule="cosine", order="stratified2d", grid=64, precision="bf16",
        description="text-to-image, 64x64 image tokens + 256 text tokens, batch 4",
    ),
    Config(
        name="c4_edit", index=3, batch=2, n_heads=32, n_kv_heads=32, head_dim=128,
        vocab=8192, prompt_len=1280, gen_len=4096, n_registers=64, n_steps=64,
        schedule="cosine", order="stratified2d", grid=64, precision="bf16",
        description="image editing: 1024 reference-image + 256 text prompt tokens, 4096 target tokens",
    ),
    Config(
        name="c5_text_semi_ar", index=4, batch=8, n_heads=32, n_kv_heads=8, head_dim=128,
        vocab=128000, prompt_len=512, gen_len=1024, n_registers=64, n_steps=128,
        schedule="semi_ar", block=32, steps_per_block=4, order="confidence", precision="bf16",
        description="semi-autoregressive text: blocks of 32, 4 sub-steps, confidence order, GQA 32/8",
    ),
)


def get_config(name_or_index) -> Config:
    for c in CONFIGS:
        if c.name == name_or_index or c.index == name_or_index:
            return c
    raise KeyError(name_or_index)
