"""ctypes binding of libmdm_sparse.so (include/mdm_sparse.h), marshalling only.

Every function has the C name and returns None or raises MdmError with the
status and the library's message.  Pointer arguments accept a torch tensor
(its data_ptr()), an int address, or None (NULL).  The library is loaded from
this package directory; if it is missing, loading raises (there is no
fallback implementation).
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmdm_sparse.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "mdm_sparse.h")

MDM_OK, MDM_E_ARG, MDM_E_SHAPE, MDM_E_CAPACITY, MDM_E_HIP, MDM_E_UNSUPPORTED, MDM_E_DEVICE = 0, -1, -2, -3, -4, -5, -6
MDM_BF16, MDM_FP32 = 0, 1
MDM_SELECT_ORDER, MDM_SELECT_CONFIDENCE = 0, 1


class MdmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_string(status)}: {msg}")
        self.status = status


class MdmConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("n_registers", ctypes.c_int32),
        ("max_decode", ctypes.c_int32),
        ("precision", ctypes.c_int32),
        ("accurate_conf", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
    ]


class MdmBuffers(ctypes.Structure):
    _fields_ = [
        ("tq", ctypes.c_void_p),
        ("tk", ctypes.c_void_p),
        ("tv", ctypes.c_void_p),
        ("w_vocab", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("cache_pos", ctypes.c_void_p),
        ("cache_tok", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MdmUpperLayers(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("w_upper", ctypes.c_void_p),
        ("k_cache_upper", ctypes.c_void_p),
        ("v_cache_upper", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MdmBlockAttnShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_rows", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SIGS = {
    "mdm_cache_slots": (ctypes.c_size_t, [ctypes.POINTER(MdmConfig)]),
    "mdm_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MdmConfig)]),
    "mdm_element_bytes": (ctypes.c_size_t, [ctypes.POINTER(MdmConfig)]),
    "mdm_sparse_step_init": (_I32, [ctypes.POINTER(_P), ctypes.POINTER(MdmConfig), ctypes.POINTER(MdmBuffers), _P]),
    "mdm_set_stream": (_I32, [_P, _P]),
    "mdm_kv_append": (_I32, [_P, _P, _P, _I64, _I32]),
    "mdm_step_attention": (_I32, [_P, _P, _P, _I64, _I32, _P, _I64, _I32, _P]),
    "mdm_subset_logits_confidence": (_I32, [_P, _P, _I64, _I32, _P, _P, _P]),
    "mdm_unmask_select": (_I32, [_P, _P, _I64, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P]),
    "mdm_order_step": (_I32, [_P, _I32, _P, _I64, _I32, _I32, _P, _P, _P, _P, _P]),
    "mdm_sparse_step_reset": (_I32, [_P]),
    "mdm_cache_len": (_I32, [_P]),
    "mdm_cache_rewind": (_I32, [_P, _I32]),
    "mdm_device_status": (_I32, [_P]),
    "mdm_set_decision_trace": (_I32, [_P, _P]),
    "mdm_decision_counts": (_I32, [_P, ctypes.POINTER(_I64)]),
    "mdm_sparse_step_destroy": (None, [_P]),
    "mdm_last_error": (ctypes.c_char_p, [_P]),
    "mdm_status_string": (ctypes.c_char_p, [_I32]),
    "mdm_upper_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MdmConfig)]),
    "mdm_attach_upper_layers": (_I32, [_P, ctypes.POINTER(MdmUpperLayers)]),
    "mdm_layer_project": (_I32, [_P, _I32, _P, _I64, _P, _I64, _I32, _P, _I64, _I32]),
    "mdm_layer_attention": (_I32, [_P, _I32, _I32, _I32, _P]),
    "mdm_block_attention_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MdmBlockAttnShape)]),
    "mdm_block_attention": (_I32, [ctypes.POINTER(MdmBlockAttnShape), _P, _P, _P, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]),
    "mdm_block_attention_static": (_I32, [ctypes.POINTER(MdmBlockAttnShape), _P, _P, _P, _P, _P, _P, _P]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises OSError if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise OSError(f"{path} not found: build it with `python -m masked_discrete_diffusion_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, ctypes.c_void_p):
        return x.value
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def status_string(status: int) -> str:
    return load().mdm_status_string(status).decode()


def _check(status: int, ctx=None):
    if status != MDM_OK:
        msg = load().mdm_last_error(ctx).decode()
        raise MdmError(status, msg)


def mdm_cache_slots(cfg: MdmConfig) -> int:
    return load().mdm_cache_slots(ctypes.byref(cfg))


def mdm_workspace_bytes(cfg: MdmConfig) -> int:
    return load().mdm_workspace_bytes(ctypes.byref(cfg))


def mdm_element_bytes(cfg: MdmConfig) -> int:
    return load().mdm_element_bytes(ctypes.byref(cfg))


def mdm_sparse_step_init(cfg: MdmConfig, bufs: MdmBuffers, stream=None):
    ctx = ctypes.c_void_p()
    _check(load().mdm_sparse_step_init(ctypes.byref(ctx), ctypes.byref(cfg), ctypes.byref(bufs), _ptr(stream)))
    return ctx


def mdm_set_stream(ctx, stream):
    _check(load().mdm_set_stream(ctx, _ptr(stream)), ctx)


def mdm_kv_append(ctx, tok, pos, stride: int, n: int):
    _check(load().mdm_kv_append(ctx, _ptr(tok), _ptr(pos), stride, n), ctx)


def mdm_step_attention(ctx, d_tok, d_pos, d_stride: int, n_new_cached: int, c_pos, c_stride: int,
                       n_decode: int, out):
    _check(load().mdm_step_attention(ctx, _ptr(d_tok), _ptr(d_pos), d_stride, n_new_cached, _ptr(c_pos),
                                     c_stride, n_decode, _ptr(out)), ctx)


def mdm_subset_logits_confidence(ctx, h, h_batch_stride: int, n_decode: int, conf, token, logits=None):
    _check(load().mdm_subset_logits_confidence(ctx, _ptr(h), h_batch_stride, n_decode, _ptr(conf), _ptr(token),
                                               _ptr(logits)), ctx)


def mdm_unmask_select(ctx, cand_pos, cand_stride: int, conf, token, n_cand: int, n_select: int, mode: int,
                      out_tok, out_pos, rem_pos=None, seq_tokens=None):
    _check(load().mdm_unmask_select(ctx, _ptr(cand_pos), cand_stride, _ptr(conf), _ptr(token), n_cand, n_select,
                                    mode, _ptr(out_tok), _ptr(out_pos), _ptr(rem_pos), _ptr(seq_tokens)), ctx)


def mdm_order_step(ctx, n_new_cached: int, c_pos, c_stride: int, n_decode: int, commit: bool, out, conf, token,
                   seq_tokens=None, logits=None):
    _check(load().mdm_order_step(ctx, n_new_cached, _ptr(c_pos), c_stride, n_decode, 1 if commit else 0, _ptr(out),
                                 _ptr(conf), _ptr(token), _ptr(seq_tokens), _ptr(logits)), ctx)


def mdm_sparse_step_reset(ctx):
    _check(load().mdm_sparse_step_reset(ctx), ctx)


def mdm_cache_len(ctx) -> int:
    return load().mdm_cache_len(ctx)


def mdm_cache_rewind(ctx, new_len: int):
    _check(load().mdm_cache_rewind(ctx, new_len), ctx)


def mdm_device_status(ctx):
    _check(load().mdm_device_status(ctx), ctx)


def mdm_set_decision_trace(ctx, trace):
    _check(load().mdm_set_decision_trace(ctx, _ptr(trace)), ctx)


def mdm_decision_counts(ctx):
    """(rows re-scored beyond the candidates, rows that re-scored whole tiles,
    rows whose two best exact logits are within twice the re-score bound)."""
    out = (_I64 * 3)()
    _check(load().mdm_decision_counts(ctx, out), ctx)
    return tuple(int(x) for x in out)


def mdm_sparse_step_destroy(ctx):
    load().mdm_sparse_step_destroy(ctx)


def mdm_last_error(ctx=None) -> str:
    return load().mdm_last_error(ctx).decode()


def mdm_block_attention_workspace_bytes(shape: MdmBlockAttnShape) -> int:
    return load().mdm_block_attention_workspace_bytes(ctypes.byref(shape))


def mdm_block_attention(shape: MdmBlockAttnShape, q, k, v, blocks, n_clean_blocks, out, workspace,
                        workspace_bytes: int, stream=None):
    _check(load().mdm_block_attention(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(blocks),
                                      _ptr(n_clean_blocks), _ptr(out), _ptr(workspace), workspace_bytes,
                                      _ptr(stream)))


def mdm_block_attention_static(shape: MdmBlockAttnShape, q, k, v, blocks, n_clean_blocks, out, stream=None):
    _check(load().mdm_block_attention_static(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(blocks),
                                             _ptr(n_clean_blocks), _ptr(out), _ptr(stream)))


def mdm_upper_workspace_bytes(cfg: MdmConfig) -> int:
    return load().mdm_upper_workspace_bytes(ctypes.byref(cfg))


def mdm_attach_upper_layers(ctx, up: MdmUpperLayers):
    _check(load().mdm_attach_upper_layers(ctx, ctypes.byref(up)), ctx)


def mdm_layer_project(ctx, layer: int, h_prev, h_batch_stride: int, d_pos, d_stride: int, n_new_cached: int,
                      c_pos, c_stride: int, n_decode: int):
    _check(load().mdm_layer_project(ctx, layer, _ptr(h_prev), h_batch_stride, _ptr(d_pos), d_stride, n_new_cached,
                                    _ptr(c_pos), c_stride, n_decode), ctx)


def mdm_layer_attention(ctx, layer: int, n_new_cached: int, n_decode: int, out):
    _check(load().mdm_layer_attention(ctx, layer, n_new_cached, n_decode, _ptr(out)), ctx)
