"""The fused order step (mdm_order_step) against the separate calls it stands
for (mdm_kv_append, mdm_step_attention, mdm_subset_logits_confidence,
mdm_unmask_select in order mode).  The same seeded workload run both ways
must agree bit for bit: every step's attention output, confidence, token and
screened logits, the final sequence, the cache (keys, values, positions,
token ids) and the cache length.  The oracle parity of the fused path itself
is covered by the generation tests, which run it by default on these
workloads."""

import numpy as np
import pytest

from mdm_inputs import get_config, make_workload
from small_workloads import gpu_small_bf16, gpu_small_d128, gpu_wide_fixed

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run(wl, fused, accurate, keep_o, keep_logits):
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    run = SparseStepRunner(wl, device="cuda", fused=fused, accurate_conf=accurate)
    assert run.fused == fused
    recs, seq = run.generate_recorded(keep_o=keep_o, keep_logits=keep_logits)
    torch.cuda.synchronize()
    cache = [t.cpu().numpy().copy() for t in (run.k_cache, run.v_cache, run.cache_pos, run.cache_tok)]
    n = L.mdm_cache_len(run.ctx)
    run.close()
    return recs, seq, cache, n


CASES = [
    ("bf16_d64", gpu_small_bf16, False),
    ("bf16_d128", gpu_small_d128, False),
    ("bf16_d128_accurate", gpu_small_d128, True),      # the attention also writes the lo half
    ("wide_fixed", gpu_wide_fixed, False),               # 512-column screen tiles
    ("c3_t2i_4k", lambda: get_config("c3_t2i_4k"), False),
]


@pytest.mark.parametrize("name,cfgfn,accurate", CASES, ids=[c[0] for c in CASES])
def test_fused_order_step_matches_separate_calls(name, cfgfn, accurate):
    cfg = cfgfn()
    _say(f"fused order step vs separate calls: {name}")
    wl = make_workload(cfg)
    n = cfg.n_steps
    small = cfg.gen_len * cfg.batch <= 4096
    keep_o = list(range(n)) if small else [0, 1, n // 2, n - 2, n - 1]
    keep_logits = keep_o if small else [0, n - 1]
    fa = _run(wl, True, accurate, keep_o, keep_logits)
    sa = _run(wl, False, accurate, keep_o, keep_logits)
    for rf, rs in zip(fa[0], sa[0]):
        k = rf["k"]
        for key in ("conf", "token", "sel_pos", "sel_tok", "o", "logits"):
            if key in rs:
                assert np.array_equal(rf[key], rs[key]), f"step {k}: {key} differs"
    assert np.array_equal(fa[1], sa[1]), "final sequences differ"
    for what, x, y in zip(("keys", "values", "positions", "token ids"), fa[2], sa[2]):
        assert np.array_equal(x, y), f"cache {what} differ"
    assert fa[3] == sa[3], "cache lengths differ"


def test_order_step_rejects_what_it_cannot_fuse():
    """Host-side checks of the fused call: the D rows must be the rows of the
    preceding commit; the fp32 precision takes the separate calls."""
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    from small_workloads import gpu_small_fp32
    cfg = gpu_small_d128()
    _say("fused order step argument checks: gpu_small_d128")
    wl = make_workload(cfg)
    run = SparseStepRunner(wl, device="cuda")
    run.prefill()
    st = run.plan[0]
    c_ptr, c_stride = run._c_src(st)
    with pytest.raises(L.MdmError) as e:           # nothing committed since the prompt's append
        L.mdm_order_step(run.ctx, 3, c_ptr, c_stride, st.n_c, True, run.out, run.conf, run.token)
    assert e.value.status == L.MDM_E_ARG
    L.mdm_order_step(run.ctx, 0, c_ptr, c_stride, st.n_c, True, run.out, run.conf, run.token)
    with pytest.raises(L.MdmError) as e:           # the commit was of st.n_c rows, not st.n_c + 1
        L.mdm_order_step(run.ctx, st.n_c + 1, c_ptr, c_stride, 1, False, run.out, run.conf, run.token)
    assert e.value.status == L.MDM_E_ARG
    torch.cuda.synchronize()
    L.mdm_device_status(run.ctx)
    run.close()
    wl32 = make_workload(gpu_small_fp32())
    run32 = SparseStepRunner(wl32, device="cuda")
    assert not run32.fused
    with pytest.raises(L.MdmError) as e:
        L.mdm_order_step(run32.ctx, 0, None, 0, 0, False, run32.out, None, None)
    assert e.value.status == L.MDM_E_UNSUPPORTED
    run32.close()


def test_order_step_without_decode_rows_is_the_attention_alone():
    """n_decode = 0: the fused call runs the attention only (no logits, no
    commit), and its output is that of mdm_step_attention on the same state."""
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    cfg = gpu_small_d128()
    _say("fused order step without decode rows: gpu_small_d128")
    wl = make_workload(cfg)
    run = SparseStepRunner(wl, device="cuda")
    run.prefill()
    st = run.plan[0]
    c_ptr, c_stride = run._c_src(st)
    L.mdm_order_step(run.ctx, 0, c_ptr, c_stride, st.n_c, True, run.out, run.conf, run.token, run.seq_tokens)
    n_q = st.n_c + cfg.n_registers
    rows = cfg.batch * n_q * cfg.hidden
    length = L.mdm_cache_len(run.ctx)
    run.out.fill_(float("nan"))
    L.mdm_order_step(run.ctx, st.n_c, None, 0, 0, True, run.out, None, None)
    torch.cuda.synchronize()
    fused = run.out[:rows].clone()
    assert L.mdm_cache_len(run.ctx) == length              # nothing committed
    run.out.fill_(float("nan"))
    # the same D rows through the separate call (their queries are the kept ones)
    d_tok = run.token[:cfg.batch * st.n_c].view(cfg.batch, st.n_c).clone()
    d_pos = run.order[:, st.c_off:st.c_off + st.n_c].contiguous()
    L.mdm_step_attention(run.ctx, d_tok, d_pos, st.n_c, st.n_c, None, 0, 0, run.out)
    torch.cuda.synchronize()
    assert torch.isfinite(fused).all()
    assert torch.equal(fused, run.out[:rows])
    L.mdm_device_status(run.ctx)
    run.close()


def test_fused_generation_repeats_bit_for_bit():
    """Two fused generations on one context (reset in between) agree bit for
    bit in every step's output, confidence and token and in the sequence."""
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    cfg = gpu_small_d128()
    _say("fused determinism: gpu_small_d128")
    wl = make_workload(cfg)
    run = SparseStepRunner(wl, device="cuda")
    steps = list(range(cfg.n_steps))
    a, sa = run.generate_recorded(keep_o=steps)
    b, sb = run.generate_recorded(keep_o=steps)
    run.close()
    assert np.array_equal(sa, sb)
    for x, y in zip(a, b):
        for key in ("o", "conf", "token"):
            assert np.array_equal(x[key], y[key]), f"step {x['k']}: {key} differs"
