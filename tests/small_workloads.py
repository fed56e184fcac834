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


def reduced(name, **kw):
    """A named workload with fewer steps/positions (same head shapes)."""
    return get_config(name).replace(**kw)


def workload(cfg, tables=True):
    return make_workload(cfg, tables=tables)
