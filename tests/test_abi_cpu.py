"""The C ABI on the CPU: the library loads, exports every function the header
declares, sizes buffers, and rejects bad arguments on the host before any GPU
call.  No compute call is made here."""

import ctypes
import os
import re

import pytest

from masked_discrete_diffusion_amd import _lib as L

HEADERS = [os.path.join(os.path.dirname(L.HEADER_PATH), f) for f in os.listdir(os.path.dirname(L.HEADER_PATH))
           if f.endswith(".h")]


def _declared():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(mdm_\w+)\s*\(", text))
    return names


def _cfg(**kw):
    base = dict(batch=2, n_heads=4, n_kv_heads=2, head_dim=64, vocab=512, seq_len=100, n_registers=8,
                max_decode=16, precision=L.MDM_BF16, accurate_conf=0, rope_theta=10000.0)
    base.update(kw)
    return L.MdmConfig(**base)


def test_library_exports_every_declared_symbol():
    lib = L.load()
    names = _declared()
    assert {"mdm_sparse_step_init", "mdm_kv_append", "mdm_step_attention",
            "mdm_subset_logits_confidence"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(L._SIGS) == names          # the binding covers exactly the header


def test_sizes():
    c = _cfg()
    assert L.mdm_cache_slots(c) == 128                       # 100 rounded up to 64
    assert L.mdm_element_bytes(c) == 2
    assert L.mdm_element_bytes(_cfg(precision=L.MDM_FP32)) == 4
    ws = L.mdm_workspace_bytes(c)
    assert ws > 0 and ws % 256 == 0
    assert L.mdm_workspace_bytes(_cfg(accurate_conf=1)) > ws  # room for the lo half of h


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), L.MDM_E_ARG),
    (dict(n_heads=6, n_kv_heads=4), L.MDM_E_ARG),
    (dict(n_registers=-1), L.MDM_E_ARG),
    (dict(max_decode=0), L.MDM_E_ARG),
    (dict(max_decode=101), L.MDM_E_ARG),
    (dict(precision=7), L.MDM_E_ARG),
    (dict(rope_theta=float("nan")), L.MDM_E_ARG),
    (dict(head_dim=96), L.MDM_E_UNSUPPORTED),
])
def test_init_rejects_bad_configs(kw, status):
    c = _cfg(**kw)
    assert L.mdm_cache_slots(c) == 0 or status == L.MDM_E_UNSUPPORTED
    with pytest.raises(L.MdmError) as e:
        L.mdm_sparse_step_init(c, L.MdmBuffers())
    assert e.value.status == status
    assert L.mdm_last_error(None)


def test_init_rejects_missing_buffers_and_small_workspace():
    c = _cfg()
    with pytest.raises(L.MdmError) as e:
        L.mdm_sparse_step_init(c, L.MdmBuffers())
    assert e.value.status == L.MDM_E_ARG
    fake = 1 << 20                                    # never dereferenced: rejected first
    b = L.MdmBuffers(tq=fake, tk=fake, tv=fake, w_vocab=fake, k_cache=fake, v_cache=fake,
                     cache_pos=fake, cache_tok=fake, workspace=fake, workspace_bytes=16)
    with pytest.raises(L.MdmError) as e:
        L.mdm_sparse_step_init(c, b)
    assert e.value.status == L.MDM_E_SHAPE
    b.workspace_bytes = L.mdm_workspace_bytes(c)
    b.workspace = fake + 8
    with pytest.raises(L.MdmError) as e:
        L.mdm_sparse_step_init(c, b)
    assert e.value.status == L.MDM_E_ARG


def test_calls_on_null_context_fail_cleanly():
    null = ctypes.c_void_p()
    for fn, args in [(L.mdm_kv_append, (None, None, 0, 1)),
                     (L.mdm_step_attention, (None, None, 0, 0, None, 0, 0, None)),
                     (L.mdm_subset_logits_confidence, (None, 0, 1, None, None)),
                     (L.mdm_unmask_select, (None, 0, None, None, 1, 1, 0, None, None)),
                     (L.mdm_order_step, (0, None, 0, 1, True, None, None, None)),
                     (L.mdm_sparse_step_reset, ()),
                     (L.mdm_device_status, ())]:
        with pytest.raises(L.MdmError) as e:
            fn(null, *args)
        assert e.value.status == L.MDM_E_ARG
    assert L.mdm_cache_len(null) == -1
    assert L.status_string(L.MDM_E_CAPACITY) == "MDM_E_CAPACITY"


def test_upper_layer_calls_validate_on_the_host():
    null = ctypes.c_void_p()
    for fn, args in [(L.mdm_attach_upper_layers, (L.MdmUpperLayers(),)),
                     (L.mdm_layer_project, (2, None, 0, None, 0, 0, None, 0, 0)),
                     (L.mdm_layer_attention, (2, 0, 0, None))]:
        with pytest.raises(L.MdmError) as e:
            fn(null, *args)
        assert e.value.status == L.MDM_E_ARG
    c = _cfg()
    ub = L.mdm_upper_workspace_bytes(c)
    assert ub > 0 and ub % 256 == 0
    assert L.mdm_upper_workspace_bytes(_cfg(precision=L.MDM_FP32)) == 0    # bf16 only


def test_block_attention_validates_on_the_host():
    fake = 1 << 20                                    # never dereferenced: rejected first
    ok = dict(batch=2, n_rows=300, n_heads=4, n_kv_heads=2, head_dim=128)
    shape = L.MdmBlockAttnShape(**ok)
    need = L.mdm_block_attention_workspace_bytes(shape)
    assert need == 2 * 5 * 2 * 4                      # [B][ceil(n/64)][2] int32
    cases = [
        (dict(ok, n_heads=3), fake, need, L.MDM_E_ARG),
        (dict(ok, n_rows=0), fake, need, L.MDM_E_ARG),
        (dict(ok, head_dim=64), fake, need, L.MDM_E_UNSUPPORTED),
        (dict(ok, n_rows=16385), fake, need, L.MDM_E_UNSUPPORTED),
        (ok, None, need, L.MDM_E_ARG),
        (ok, fake + 8, need, L.MDM_E_ARG),              # q misaligned
        (ok, fake, need - 4, L.MDM_E_SHAPE),
    ]
    for kw, q, ws, status in cases:
        with pytest.raises(L.MdmError) as e:
            L.mdm_block_attention(L.MdmBlockAttnShape(**kw), q, fake, fake, fake, fake, fake, fake, ws, None)
        assert e.value.status == status, (kw, q, ws)
    assert L.mdm_block_attention_workspace_bytes(L.MdmBlockAttnShape(**dict(ok, n_heads=3))) == 0


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with a message before any
    device work."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
