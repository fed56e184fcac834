"""Sparse masked-discrete-diffusion sampling step on MI355X (gfx950).

The compute path is the HIP library libmdm_sparse.so (C ABI in
include/mdm_sparse.h); ``_lib`` binds it with ctypes and ``sampler`` drives
the per-step calls over PyTorch-allocated device buffers.
"""

from . import _lib  # noqa: F401
from ._lib import MdmError  # noqa: F401

__all__ = ["_lib", "MdmError"]
