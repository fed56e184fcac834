"""Small seeded workloads for oracle and parity tests (shapes only; data comes
from mdm_inputs)."""

from mdm_inputs import Config, get_config, make_workload


def tiny_bf16(index=100, **kw):
    base = dict(name="tiny_bf16", index=index, batch=2, n_heads=4, n_kv_heads=2, head_dim=16,
                vocab=64, prompt_len=6, gen_len=16, n_registers=3, n_steps=4,
                schedule="fixed", per_step=4, order="random", precision="bf16")
    base.update(kw)
    return Config(**base)


def tiny_semi_ar(index=101, **kw):
    base = dict(name="tiny_semi_ar", index=index, batch=3, n_heads=4, n_kv_heads=1, head_dim=16,
                vocab=48, prompt_len=5, gen_len=16, n_registers=2, n_steps=8,
                schedule="semi_ar", block=8, steps_per_block=4, order="confidence",
                precision="bf16")
    base.update(kw)
    return Config(**base)


def tiny_infill(index=102, **kw):
    """Semi-AR text infilling: three masked spans inside the sequence, blocks in
    a seeded random order."""
    base = dict(name="tiny_infill", infill_spans=3, block_order="random", block=4, steps_per_block=2)
    base.update(kw)
    return tiny_semi_ar(index=index, **base)


def reduced(name, **kw):
    """A named workload with fewer steps/positions (same head shapes)."""
    return get_config(name).replace(**kw)


def workload(cfg, tables=True):
    return make_workload(cfg, tables=tables)


# Shapes the HIP path supports (head_dim 64/128), small enough for a live oracle,
# ragged on purpose: key counts and row counts are not multiples of the tiles.
def gpu_small_bf16(index=110, **kw):
    base = dict(name="gpu_small_bf16", index=index, batch=2, n_heads=4, n_kv_heads=2, head_dim=64,
                vocab=1000, prompt_len=40, gen_len=96, n_registers=8, n_steps=6,
                schedule="fixed", per_step=16, order="random", precision="bf16")
    base.update(kw)
    return Config(**base)


def gpu_small_d128(index=111, **kw):
    base = dict(name="gpu_small_d128", index=index, batch=2, n_heads=8, n_kv_heads=8, head_dim=128,
                vocab=700, prompt_len=70, gen_len=144, n_registers=64, n_steps=8,
                schedule="cosine", order="stratified2d", grid=12, precision="bf16")
    base.update(kw)
    return Config(**base)


def gpu_small_semi_ar(index=112, **kw):
    base = dict(name="gpu_small_semi_ar", index=index, batch=3, n_heads=8, n_kv_heads=2, head_dim=128,
                vocab=3000, prompt_len=33, gen_len=64, n_registers=5, n_steps=16,
                schedule="semi_ar", block=16, steps_per_block=4, order="confidence", precision="bf16")
    base.update(kw)
    return Config(**base)


def gpu_small_fp32(index=113, **kw):
    return gpu_small_d128(index=index, name="gpu_small_fp32", precision="fp32", **kw)


# Vocabularies large enough for the 512-column screen tiles (at least 224
# of them): semi-autoregressive (hi/lo screening, 64- and 128-row tiles) and a
# fixed schedule (hi only, 128-row tiles).  hidden 256 keeps the oracle fast.
def gpu_wide_semi_ar(index=115, **kw):
    base = dict(name="gpu_wide_semi_ar", index=index, batch=8, n_heads=2, n_kv_heads=1, head_dim=128,
                vocab=120000, prompt_len=24, gen_len=32, n_registers=4, n_steps=8,
                schedule="semi_ar", block=16, steps_per_block=4, order="confidence", precision="bf16")
    base.update(kw)
    return Config(**base)


# Semi-AR blocks of 24 decoded 6 at a time over 8 sequences: steps of 192
# and 144 rows take three and three 64-row tiles of the wide screen (hi + lo).
def gpu_wide_semi_ar_192(index=123, **kw):
    base = dict(name="gpu_wide_semi_ar_192", index=index, batch=8, n_heads=2, n_kv_heads=1, head_dim=128,
                vocab=120000, prompt_len=24, gen_len=48, n_registers=4, n_steps=8,
                schedule="semi_ar", block=24, steps_per_block=4, order="confidence", precision="bf16")
    base.update(kw)
    return Config(**base)


def gpu_wide_fixed(index=116, **kw):
    base = dict(name="gpu_wide_fixed", index=index, batch=8, n_heads=2, n_kv_heads=2, head_dim=128,
                vocab=115000, prompt_len=30, gen_len=32, n_registers=4, n_steps=2,
                schedule="fixed", per_step=16, order="random", precision="bf16")
    base.update(kw)
    return Config(**base)


# Blocks of five query chunks (the fifth split over four wavefronts): 3 x 32
# heads, 100 rows decoded per step, so steps 2 and 3 have 100 + 100 + 64
# query rows = 10 chunks per head in two groups of five.
def gpu_five_chunks(index=118, **kw):
    base = dict(name="gpu_five_chunks", index=index, batch=3, n_heads=32, n_kv_heads=32, head_dim=128,
                vocab=300, prompt_len=16, gen_len=300, n_registers=64, n_steps=3,
                schedule="fixed", per_step=100, order="random", precision="bf16")
    base.update(kw)
    return Config(**base)


# Text variants on the HIP path: infilling (four masked spans inside the
# sequence) with semi-AR blocks decoded in a seeded random order.
def gpu_text_infill(index=117, **kw):
    base = dict(name="gpu_text_infill", infill_spans=4, block_order="random")
    base.update(kw)
    return gpu_small_semi_ar(index=index, **base)


# Training-form (block-mask) attention: ragged block boundaries, grouped
# heads, rows in block order and shuffled, fewer rows than one key tile.
def ba_small(index=130, **kw):
    from mdm_inputs.training import TrainAttnConfig
    base = dict(name="ba_small", index=index, batch=2, n_heads=4, n_kv_heads=2, head_dim=128, prompt_len=37,
                gen_len=300, n_registers=5, clean_blocks=3, masked_blocks=4)
    base.update(kw)
    return TrainAttnConfig(**base)


BA_CASES = {
    "ragged_gqa2": lambda: ba_small(),
    "shuffled_rows": lambda: ba_small(index=131, n_heads=2, n_kv_heads=2, shuffle_rows=True),
    "under_one_tile_gqa8": lambda: ba_small(index=132, batch=3, n_heads=8, n_kv_heads=1, prompt_len=5,
                                            gen_len=30, n_registers=3, clean_blocks=2, masked_blocks=2),
    "aligned_text_gqa4": lambda: ba_small(index=133, n_heads=8, n_kv_heads=2, prompt_len=64, gen_len=256,
                                          n_registers=16, clean_blocks=4, masked_blocks=4),
    "all_masked": lambda: ba_small(index=134, n_heads=2, n_kv_heads=1, prompt_len=20, gen_len=150,
                                   n_registers=7, clean_blocks=0, masked_blocks=5, mask_ratio=1.0),
    "single_head_long": lambda: ba_small(index=135, batch=1, n_heads=1, n_kv_heads=1, prompt_len=100,
                                         gen_len=1500, n_registers=20, clean_blocks=6, masked_blocks=3),
}


# Two attention layers (layer 2 projects layer 1's outputs; its own cache).
def tiny_two_layer(index=103, **kw):
    base = dict(name="tiny_two_layer", layers=2)
    base.update(kw)
    return tiny_bf16(index=index, **base)


def gpu_two_layer(index=118, **kw):
    base = dict(name="gpu_two_layer", layers=2)
    base.update(kw)
    return gpu_small_bf16(index=index, head_dim=128, **base)


def gpu_two_layer_semi_ar(index=119, **kw):
    base = dict(name="gpu_two_layer_semi_ar", layers=2, n_heads=4, n_kv_heads=2, vocab=1200)
    base.update(kw)
    return gpu_small_semi_ar(index=index, **base)


# Two layers at the production head shape (32 heads x 128, so 12288
# projection rows = 24 tiles of 512 columns) with a 1100-token prompt: the
# prefill projection of 1116 rows takes the projection's wide tiles (9 row
# tiles x 24 = 216 blocks), the decode steps the 128-column tiles.
def gpu_two_layer_wide(index=122, **kw):
    base = dict(name="gpu_two_layer_wide", index=index, batch=1, n_heads=32, n_kv_heads=32, head_dim=128,
                vocab=1000, prompt_len=1100, gen_len=96, n_registers=16, n_steps=3,
                schedule="fixed", per_step=32, order="random", precision="bf16", layers=2)
    base.update(kw)
    return Config(**base)


# The bf16 screen's row tilings and hidden splits on one 8192-column
# vocabulary: a cosine schedule over 600 positions in 8 steps decodes
# 12..117 rows per sequence, 36..351 rows per step over 3 sequences.
def gpu_screen_regimes(index=120, **kw):
    base = dict(name="gpu_screen_regimes", index=index, batch=3, n_heads=2, n_kv_heads=2, head_dim=128,
                vocab=8192, prompt_len=20, gen_len=600, n_registers=16, n_steps=8,
                schedule="cosine", order="random", precision="bf16")
    base.update(kw)
    return Config(**base)


# The production decision kernel's shape (hidden 4096 = 32 heads x 128) with a
# 2048-column vocabulary (16 tiles of 128) and 32 decoded rows per step; the
# decision tests rewrite its head so that columns tie.
def gpu_decide_dup(index=121, **kw):
    base = dict(name="gpu_decide_dup", index=index, batch=2, n_heads=32, n_kv_heads=8, head_dim=128,
                vocab=2048, prompt_len=20, gen_len=48, n_registers=4, n_steps=3,
                schedule="fixed", per_step=16, order="random", precision="bf16")
    base.update(kw)
    return Config(**base)
