"""Fused Dynamic Tanh (DyT) layer for AMD Instinct MI355X (gfx950).

y = gamma * tanh(alpha * x) + beta over an M x N row-major activation and its
backward (dx, dgamma, dbeta, dalpha), also with the residual add fused in
front (h = x + r, y = DyT(h)), computed by hand-written HIP kernels
behind a C ABI (``include/dyt.h``, library ``libdyt.so`` in this package).
The Python functions below carry the ABI's names and only marshal tensors.
"""
from ._lib import (  # noqa: F401
    DYT_BF16,
    DYT_F16,
    DYT_F32,
    DYT_OK,
    LIB_FILE,
    DytError,
    dyt_abi_version,
    dyt_backward,
    dyt_backward_finish,
    dyt_backward_noalloc,
    dyt_backward_partials,
    dyt_backward_residual,
    dyt_backward_residual_partials,
    dyt_backward_workspace_size,
    dyt_forward,
    dyt_forward_residual,
    dyt_get_forward_plan,
    dyt_get_forward_residual_plan,
    dyt_get_plan,
    dyt_set_xcd_flip_override,
    dyt_status_string,
    dyt_xcd_hint,
    lib,
)

from .module import DyT, DyTFunction, DyTResidual, DyTResidualFunction, dyt, dyt_residual  # noqa: E402,F401

__all__ = [
    "DyT", "DyTFunction", "dyt", "DyTResidual", "DyTResidualFunction", "dyt_residual",
    "DYT_F32", "DYT_BF16", "DYT_F16", "DYT_OK", "DytError", "LIB_FILE", "lib",
    "dyt_forward", "dyt_backward", "dyt_backward_partials", "dyt_backward_finish",
    "dyt_backward_workspace_size", "dyt_backward_noalloc", "dyt_forward_residual", "dyt_backward_residual",
    "dyt_backward_residual_partials",
    "dyt_status_string", "dyt_abi_version", "dyt_get_plan", "dyt_get_forward_plan",
    "dyt_get_forward_residual_plan", "dyt_xcd_hint", "dyt_set_xcd_flip_override",
]
