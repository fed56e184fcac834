"""The allocation-free training-form attention (mdm_block_attention_static)
against the workspace entry point it varies, through the C ABI: the same
kernels, so the outputs must be identical, on two calls in a row (the second
with a smaller input, so stale ranges of the first call sit in the shared
array), and a shape beyond the array's capacity is refused before any launch."""

import numpy as np
import pytest

from mdm_inputs.training import make_train_attn_inputs
from small_workloads import ba_small

pytestmark = pytest.mark.gpu


def _tensors(inp):
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")
    return (t(inp.q), t(inp.k), t(inp.v), torch.from_numpy(inp.blocks).to("cuda"),
            torch.from_numpy(inp.n_clean).to("cuda"))


def _both(inp):
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    cfg = inp.cfg
    q, k, v, blocks, n_clean = _tensors(inp)
    shape = L.MdmBlockAttnShape(batch=cfg.batch, n_rows=cfg.n_rows, n_heads=cfg.n_heads,
                                n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim)
    stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = L.mdm_block_attention_workspace_bytes(shape)
    ws = torch.zeros(ws_bytes // 4 + 1, dtype=torch.int32, device="cuda")
    ref = torch.full((cfg.batch, cfg.n_rows, cfg.n_heads, cfg.head_dim), float("nan"), device="cuda")
    got = torch.full_like(ref, float("nan"))
    L.mdm_block_attention(shape, q, k, v, blocks, n_clean, ref, ws, ws_bytes, stream)
    L.mdm_block_attention_static(shape, q, k, v, blocks, n_clean, got, stream)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_static_ranges_match_the_workspace_entry_point_twice():
    big = make_train_attn_inputs(ba_small(index=140, batch=3, n_heads=4, n_kv_heads=2, prompt_len=60,
                                          gen_len=700, n_registers=9, clean_blocks=4, masked_blocks=5))
    small = make_train_attn_inputs(ba_small(index=141, batch=2, n_heads=2, n_kv_heads=1, prompt_len=20,
                                            gen_len=150, n_registers=5, clean_blocks=2, masked_blocks=3))
    assert small.cfg.batch * -(-small.cfg.n_rows // 64) < big.cfg.batch * -(-big.cfg.n_rows // 64)
    for inp in (big, small):
        print(f"no-alloc block attention: batch {inp.cfg.batch}, {inp.cfg.n_rows} rows", flush=True)
        ref, got = _both(inp)
        assert np.isfinite(ref).all()
        assert np.array_equal(ref, got), f"outputs differ in {int((ref != got).sum())} elements"


def test_static_ranges_refuse_a_shape_beyond_capacity():
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    # 33 sequences of 16384 rows need 33 * 256 tile ranges, over the 8192 the array holds
    shape = L.MdmBlockAttnShape(batch=33, n_rows=16384, n_heads=1, n_kv_heads=1, head_dim=128)
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    with pytest.raises(L.MdmError) as e:
        L.mdm_block_attention_static(shape, buf, buf, buf, buf, buf, buf, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == L.MDM_E_UNSUPPORTED
