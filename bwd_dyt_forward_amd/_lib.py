"""Python binding of the DyT C ABI (include/dyt.h): argument marshalling only.

Every computation runs in the HIP library ``libdyt.so``; this module only
checks tensor shapes, allocates outputs and workspace with PyTorch, and
passes device pointers and torch's current HIP stream across the ABI. There
is no CPU fallback: importing this module fails if the library is missing.
"""
from __future__ import annotations

import ctypes
import os

# torch first: libdyt.so then binds to the HIP runtime torch already loaded
# (same SONAME), so torch's streams and allocations are valid across the ABI.
import torch

from .build import LIB_PATH, source_hash

DYT_F32 = 0
DYT_BF16 = 1
DYT_F16 = 2
DYT_OK = 0
# DYT_ABI_VERSION of include/dyt.h that the signatures and DytPlan below mirror
ABI_VERSION = 7

_TORCH_TO_CODE = {torch.float32: DYT_F32, torch.bfloat16: DYT_BF16, torch.float16: DYT_F16}
_CODE_TO_TORCH = {v: k for k, v in _TORCH_TO_CODE.items()}


class DytError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {message} ({status})")
        self.status = status


class DytPlan(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_int32), ("vec", ctypes.c_int32), ("slots", ctypes.c_int32),
        ("block", ctypes.c_int32), ("rows_per_tile", ctypes.c_int64),
        ("tile_elems", ctypes.c_int64), ("col_blocks", ctypes.c_int64), ("tiles", ctypes.c_int64),
        ("fwd_grid", ctypes.c_int64), ("bwd_grid", ctypes.c_int64), ("ws_row", ctypes.c_int64),
        ("fin_grid", ctypes.c_int64), ("ws_bytes", ctypes.c_int64),
        ("flat", ctypes.c_int64), ("flat_grid", ctypes.c_int64),
        ("flat_aligned_only", ctypes.c_int64),
    ]


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int

SIGNATURES = {
    "dyt_forward": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _int, _vp]),
    "dyt_backward_workspace_size": (ctypes.c_size_t, [_i64, _i64, _int, _int]),
    "dyt_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                            _i64, _i64, _int, _int, _vp]),
    "dyt_backward_partials": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _i64, _i64,
                                     _int, _int, _vp]),
    "dyt_backward_finish": (_int, [_vp, ctypes.c_size_t, _vp, _vp, _vp, _i64, _i64, _int, _int, _vp]),
    "dyt_forward_residual": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _int, _vp]),
    "dyt_forward_strided": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp]),
    "dyt_backward_strided": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp,
                                    ctypes.c_size_t, _i64, _i64, _int, _int, _vp]),
    "dyt_backward_residual": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _i64, _i64, _int, _int, _vp]),
    "dyt_backward_residual_partials": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                              _i64, _i64, _int, _int, _vp]),
    "dyt_backward_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _int,
                                    _vp]),
    "dyt_status_string": (ctypes.c_char_p, [_int]),
    "dyt_abi_version": (_int, []),
    "dyt_build_id": (ctypes.c_char_p, []),
    "dyt_xcd_hint": (_int, [ctypes.c_void_p]),
    "dyt_set_xcd_flip_override": (_int, [_int]),
    "dyt_get_plan": (_int, [_i64, _i64, _int, _int, _int, ctypes.POINTER(DytPlan)]),
    "dyt_get_forward_plan": (_int, [_i64, _i64, _int, _int, _int, ctypes.POINTER(DytPlan)]),
    "dyt_get_forward_residual_plan": (_int, [_i64, _i64, _int, _int, ctypes.POINTER(DytPlan)]),
}


def _load(path: str = LIB_PATH, extra_flags=(), any_sources: bool = False) -> ctypes.CDLL:
    """Load the library at path, built from the current sources with the
    extra compiler flags extra_flags (a variant build), or raise; with
    any_sources, a library of this ABI built from any sources (another
    build to measure against)."""
    if not os.path.exists(path):
        raise ImportError(
            f"DyT HIP library not found at {path}; build it first "
            "(python bwd_dyt_forward_amd/build.py, or __graft_entry__.build())")
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    found = lib.dyt_abi_version()
    if found != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {found}, this binding expects {ABI_VERSION}; "
                          "rebuild the library")
    built, want = lib.dyt_build_id().decode(), source_hash(tuple(extra_flags))
    if built != want and not any_sources:
        raise ImportError(f"{path} was built from other sources (build id {built}, sources "
                          f"{want}); rebuild it (python bwd_dyt_forward_amd/build.py)")
    return lib


lib = _load()
LIB_FILE = LIB_PATH


def _check(fn: str, status: int) -> None:
    if status != DYT_OK:
        raise DytError(fn, status, lib.dyt_status_string(status).decode())


def _code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    if isinstance(dtype, str):
        return {"f32": DYT_F32, "bf16": DYT_BF16, "f16": DYT_F16}[dtype]
    try:
        return _TORCH_TO_CODE[dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {dtype}") from None


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _keep_alive_on(stream, *made: torch.Tensor) -> None:
    """Tensors this module allocated for a launch on an explicit stream other
    than torch's current one: tell the caching allocator that `stream` uses
    them, so that their memory is not handed out again (to work on the
    current stream) before the kernels on `stream` are done with it."""
    if stream is None:
        return
    cur = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        s = stream
    else:
        if int(stream) == cur.cuda_stream:
            return
        s = torch.cuda.ExternalStream(int(stream))
    if s.cuda_stream == cur.cuda_stream:
        return
    for t in made:
        if t is not None:
            t.record_stream(s)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _check_act(name: str, t: torch.Tensor, strided: bool = False) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if strided:
        if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1) or \
                (t.size(0) > 1 and t.stride(0) < t.size(1)):
            raise ValueError(f"{name} must be a 2-D [M, N] tensor with unit column stride and "
                             "row stride >= N")
    elif t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D [M, N] tensor")


def _pitch(t: torch.Tensor) -> int:
    """Row pitch in elements (N for a single row or a contiguous tensor)."""
    return t.stride(0) if t.size(0) > 1 else t.size(1)


def _check_params(N: int, device, alpha, *vecs) -> None:
    """alpha (one element) and gamma/beta (N elements each): contiguous device
    tensors of one dtype on the activations' device. The kernels dereference
    these pointers, so a host tensor must never reach the ABI."""
    for name, t in (("alpha", alpha), *(("gamma/beta", v) for v in vecs)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
            raise ValueError(f"{name} must be a tensor on {device}, like the activations")
    if alpha.numel() != 1:
        raise ValueError("alpha must hold one element")
    for v in vecs:
        if v.numel() != N or not v.is_contiguous():
            raise ValueError("gamma/beta must be contiguous with N elements")
    dts = {alpha.dtype, *(v.dtype for v in vecs)}
    if len(dts) != 1:
        raise ValueError("alpha, gamma and beta must share one dtype")


def dyt_forward(x: torch.Tensor, alpha: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor,
                y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = gamma * tanh(alpha * x) + beta on the HIP stream (async). x and y
    may be row-strided 2-D views (unit column stride); a new y is contiguous."""
    _check_act("x", x, strided=True)
    M, N = x.shape
    _check_params(N, x.device, alpha, gamma, beta)
    made_y = y is None
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _check_act("y", y, strided=True)
        if y.shape != x.shape or y.dtype != x.dtype:
            raise ValueError("y must match x in shape and dtype")
    ldx, ldy = _pitch(x), _pitch(y)
    if ldx == N and ldy == N:
        st = lib.dyt_forward(_ptr(x), _ptr(alpha), _ptr(gamma), _ptr(beta), _ptr(y), M, N,
                             _code(x.dtype), _code(alpha.dtype), _stream(stream))
        _check("dyt_forward", st)
    else:
        st = lib.dyt_forward_strided(_ptr(x), ldx, _ptr(alpha), _ptr(gamma), _ptr(beta), _ptr(y),
                                     ldy, M, N, _code(x.dtype), _code(alpha.dtype), _stream(stream))
        _check("dyt_forward_strided", st)
    if made_y:
        _keep_alive_on(stream, y)
    return y


def dyt_backward_workspace_size(M: int, N: int, x_dtype, param_dtype) -> int:
    return int(lib.dyt_backward_workspace_size(int(M), int(N), _code(x_dtype), _code(param_dtype)))


def dyt_backward(x: torch.Tensor, dy: torch.Tensor, alpha: torch.Tensor, gamma: torch.Tensor,
                 dx: torch.Tensor | None = None, dalpha: torch.Tensor | None = None,
                 dgamma: torch.Tensor | None = None, dbeta: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, stream=None):
    """Returns (dx, dalpha, dgamma, dbeta); enqueued on the HIP stream (async).
    x, dy and dx may be row-strided 2-D views (unit column stride); a new dx
    is contiguous."""
    _check_act("x", x, strided=True)
    _check_act("dy", dy, strided=True)
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    M, N = x.shape
    _check_params(N, x.device, alpha, gamma)
    pdt = alpha.dtype
    dev = x.device
    made = [t is None for t in (dx, dalpha, dgamma, dbeta, workspace)]
    if dx is None:
        dx = torch.empty((M, N), dtype=x.dtype, device=dev)
    else:
        _check_act("dx", dx, strided=True)
        if dx.shape != x.shape or dx.dtype != x.dtype:
            raise ValueError("dx must match x in shape and dtype")
    if dalpha is None:
        dalpha = torch.empty(1, dtype=pdt, device=dev)
    if dgamma is None:
        dgamma = torch.empty(N, dtype=pdt, device=dev)
    if dbeta is None:
        dbeta = torch.empty(N, dtype=pdt, device=dev)
    need = dyt_backward_workspace_size(M, N, x.dtype, pdt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    ldx, lddy, lddx = _pitch(x), _pitch(dy), _pitch(dx)
    if ldx == N and lddy == N and lddx == N:
        st = lib.dyt_backward(_ptr(x), _ptr(dy), _ptr(alpha), _ptr(gamma), _ptr(dx), _ptr(dalpha),
                              _ptr(dgamma), _ptr(dbeta), _ptr(workspace), wbytes, M, N,
                              _code(x.dtype), _code(pdt), _stream(stream))
        _check("dyt_backward", st)
    else:
        st = lib.dyt_backward_strided(_ptr(x), ldx, _ptr(dy), lddy, _ptr(alpha), _ptr(gamma),
                                      _ptr(dx), lddx, _ptr(dalpha), _ptr(dgamma), _ptr(dbeta),
                                      _ptr(workspace), wbytes, M, N, _code(x.dtype), _code(pdt),
                                      _stream(stream))
        _check("dyt_backward_strided", st)
    _keep_alive_on(stream, *(t for t, m in zip((dx, dalpha, dgamma, dbeta, workspace), made) if m))
    return dx, dalpha, dgamma, dbeta


# Bytes of the static device array dyt_backward_noalloc keeps its partial
# rows in (DYT_NOALLOC_SCRATCH_BYTES of include/dyt.h).
NOALLOC_SCRATCH_BYTES = 16 << 20


def dyt_backward_noalloc(x: torch.Tensor, dy: torch.Tensor, alpha: torch.Tensor,
                         gamma: torch.Tensor, dx: torch.Tensor, dalpha: torch.Tensor,
                         dgamma: torch.Tensor, dbeta: torch.Tensor, stream=None):
    """dyt_backward with the library's static scratch instead of a workspace:
    the caller passes every output, the call allocates nothing. Calls that
    overlap on one GPU share the scratch and race."""
    _check_act("x", x)
    _same("dy", dy, x)
    _same("dx", dx, x)
    M, N = x.shape
    _check_params(N, x.device, alpha, gamma)
    _check_params(N, x.device, dalpha, dgamma, dbeta)
    if dalpha.dtype != alpha.dtype:
        raise ValueError("dalpha, dgamma and dbeta must have the parameters' dtype")
    st = lib.dyt_backward_noalloc(_ptr(x), _ptr(dy), _ptr(alpha), _ptr(gamma), _ptr(dx),
                                  _ptr(dalpha), _ptr(dgamma), _ptr(dbeta), M, N, _code(x.dtype),
                                  _code(alpha.dtype), _stream(stream))
    _check("dyt_backward_noalloc", st)
    return dx, dalpha, dgamma, dbeta


def dyt_backward_partials(x: torch.Tensor, dy: torch.Tensor, alpha: torch.Tensor,
                          gamma: torch.Tensor, dx: torch.Tensor, workspace: torch.Tensor,
                          stream=None) -> torch.Tensor:
    """First backward pass: dx plus the float32 partial rows in workspace."""
    _check_act("x", x)
    _check_act("dy", dy)
    M, N = x.shape
    _check_params(N, x.device, alpha, gamma)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.dyt_backward_partials(_ptr(x), _ptr(dy), _ptr(alpha), _ptr(gamma), _ptr(dx),
                                   _ptr(workspace), wbytes, M, N, _code(x.dtype),
                                   _code(alpha.dtype), _stream(stream))
    _check("dyt_backward_partials", st)
    return dx


def dyt_backward_finish(workspace: torch.Tensor, M: int, N: int, x_dtype,
                        dalpha: torch.Tensor, dgamma: torch.Tensor, dbeta: torch.Tensor,
                        stream=None):
    """Second backward pass: fixed-order sums of the partial rows."""
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.dyt_backward_finish(_ptr(workspace), wbytes, _ptr(dalpha), _ptr(dgamma), _ptr(dbeta),
                                 int(M), int(N), _code(x_dtype), _code(dalpha.dtype),
                                 _stream(stream))
    _check("dyt_backward_finish", st)
    return dalpha, dgamma, dbeta


def _same(name: str, t: torch.Tensor, ref: torch.Tensor) -> None:
    _check_act(name, t)
    if t.shape != ref.shape or t.dtype != ref.dtype:
        raise ValueError(f"{name} must match {tuple(ref.shape)} {ref.dtype}")


def dyt_forward_residual(x: torch.Tensor, r: torch.Tensor, alpha: torch.Tensor,
                         gamma: torch.Tensor, beta: torch.Tensor, h: torch.Tensor | None = None,
                         y: torch.Tensor | None = None, stream=None):
    """h = x + r (rounded to x's dtype), y = gamma * tanh(alpha * h) + beta; returns (h, y)."""
    _check_act("x", x)
    _same("r", r, x)
    M, N = x.shape
    _check_params(N, x.device, alpha, gamma, beta)
    made = [h is None, y is None]
    if h is None:
        h = torch.empty_like(x)
    if y is None:
        y = torch.empty_like(x)
    st = lib.dyt_forward_residual(_ptr(x), _ptr(r), _ptr(alpha), _ptr(gamma), _ptr(beta), _ptr(h),
                                  _ptr(y), M, N, _code(x.dtype), _code(alpha.dtype),
                                  _stream(stream))
    _check("dyt_forward_residual", st)
    _keep_alive_on(stream, *(t for t, m in zip((h, y), made) if m))
    return h, y


def dyt_backward_residual(h: torch.Tensor, dy: torch.Tensor, dres: torch.Tensor,
                          alpha: torch.Tensor, gamma: torch.Tensor, dh: torch.Tensor | None = None,
                          dalpha: torch.Tensor | None = None, dgamma: torch.Tensor | None = None,
                          dbeta: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                          stream=None):
    """dh = dres + (DyT backward of dy at h); returns (dh, dalpha, dgamma, dbeta)."""
    _check_act("h", h)
    _same("dy", dy, h)
    _same("dres", dres, h)
    M, N = h.shape
    _check_params(N, h.device, alpha, gamma)
    pdt = alpha.dtype
    dev = h.device
    made = [t is None for t in (dh, dalpha, dgamma, dbeta, workspace)]
    if dh is None:
        dh = torch.empty_like(h)
    if dalpha is None:
        dalpha = torch.empty(1, dtype=pdt, device=dev)
    if dgamma is None:
        dgamma = torch.empty(N, dtype=pdt, device=dev)
    if dbeta is None:
        dbeta = torch.empty(N, dtype=pdt, device=dev)
    need = dyt_backward_workspace_size(M, N, h.dtype, pdt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.dyt_backward_residual(_ptr(h), _ptr(dy), _ptr(dres), _ptr(alpha), _ptr(gamma),
                                   _ptr(dh), _ptr(dalpha), _ptr(dgamma), _ptr(dbeta),
                                   _ptr(workspace), wbytes, M, N, _code(h.dtype), _code(pdt),
                                   _stream(stream))
    _check("dyt_backward_residual", st)
    _keep_alive_on(stream, *(t for t, m in zip((dh, dalpha, dgamma, dbeta, workspace), made) if m))
    return dh, dalpha, dgamma, dbeta


def dyt_backward_residual_partials(h: torch.Tensor, dy: torch.Tensor, dres: torch.Tensor,
                                   alpha: torch.Tensor, gamma: torch.Tensor, dh: torch.Tensor,
                                   workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """First pass of the residual backward: dh plus the partial rows in workspace."""
    _check_act("h", h)
    _same("dy", dy, h)
    _same("dres", dres, h)
    M, N = h.shape
    _check_params(N, h.device, alpha, gamma)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.dyt_backward_residual_partials(_ptr(h), _ptr(dy), _ptr(dres), _ptr(alpha),
                                            _ptr(gamma), _ptr(dh), _ptr(workspace), wbytes, M, N,
                                            _code(h.dtype), _code(alpha.dtype), _stream(stream))
    _check("dyt_backward_residual_partials", st)
    return dh


def dyt_status_string(status: int) -> str:
    return lib.dyt_status_string(int(status)).decode()


def dyt_abi_version() -> int:
    return int(lib.dyt_abi_version())


def dyt_xcd_hint(stream=None) -> int:
    """The XCD (0-7) the last XCD-weighted forward on `stream` started on, -1 if none."""
    return int(lib.dyt_xcd_hint(_stream(stream)))


def dyt_set_xcd_flip_override(flip: int) -> None:
    """Force the forward's XCD parity (0 or 1) for later launches; -1 follows the hint."""
    _check("dyt_set_xcd_flip_override", lib.dyt_set_xcd_flip_override(int(flip)))


def dyt_get_plan(M: int, N: int, x_dtype, param_dtype, vector_access: bool = True) -> dict:
    """The backward's plan (tiles, grid, workspace layout) and the forward's grid."""
    p = DytPlan()
    st = lib.dyt_get_plan(int(M), int(N), _code(x_dtype), _code(param_dtype),
                          1 if vector_access else 0, ctypes.byref(p))
    _check("dyt_get_plan", st)
    return {name: getattr(p, name) for name, _ in DytPlan._fields_}


def dyt_get_forward_residual_plan(M: int, N: int, x_dtype, param_dtype) -> dict:
    """The residual-fused forward's plan (its tiles or flat walk, and grid)."""
    p = DytPlan()
    st = lib.dyt_get_forward_residual_plan(int(M), int(N), _code(x_dtype), _code(param_dtype),
                                           ctypes.byref(p))
    _check("dyt_get_forward_residual_plan", st)
    return {name: getattr(p, name) for name, _ in DytPlan._fields_}


def dyt_get_forward_plan(M: int, N: int, x_dtype, param_dtype, vector_access: bool = True) -> dict:
    """The forward's plan (its tiles and grid; backward-only fields are 0)."""
    p = DytPlan()
    st = lib.dyt_get_forward_plan(int(M), int(N), _code(x_dtype), _code(param_dtype),
                                  1 if vector_access else 0, ctypes.byref(p))
    _check("dyt_get_forward_plan", st)
    return {name: getattr(p, name) for name, _ in DytPlan._fields_}
