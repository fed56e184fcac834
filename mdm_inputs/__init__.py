"""Seeded synthetic workloads for the sparse masked-diffusion sampling step.

This package is the only code shared by the CPU oracle (``oracle/``) and the
HIP path (``masked_discrete_diffusion_amd``).  It draws random numbers and
lays out the workload definition (shapes, per-step decode counts, the
pre-generated unmask order); it holds none of the step's arithmetic
(no RoPE, no attention, no logits, no selection).
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .generate import (  # noqa: F401
    Workload,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    make_workload,
    cosine_counts,
    stratified_order_2d,
)
