"""Plain fp64 CPU oracle for the fused Dynamic Tanh (DyT) layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The HIP library
never calls it and has no CPU fallback; this file shares no code, constant
or helper with it.

What is computed
----------------
The DyT layer (the one the Liger-Kernel pull request "fix(dyt): use a 1D
grid and tile small-width rows" fixes; its Summary names alpha, gamma,
beta and their gradients dalpha, dgamma, dbeta) is, for an M x N row-major
activation x, a scalar alpha and per-column gamma and beta:

    y[i, j]   = gamma[j] * tanh(alpha * x[i, j]) + beta[j]

and its backward, for an upstream gradient dy of the same shape, is the
chain rule of that forward, with s = sech^2(alpha * x) = 1 - tanh^2(alpha x):

    dx[i, j]  = dy[i, j] * gamma[j] * alpha * s[i, j]
    dgamma[j] = sum_i dy[i, j] * tanh(alpha * x[i, j])
    dbeta[j]  = sum_i dy[i, j]
    dalpha    = sum_{i, j} dy[i, j] * gamma[j] * x[i, j] * s[i, j]

The backward takes x (not y) and recomputes tanh from it: the pull
request's Summary ("Padding" bullet) reasons about tanh(inf * 0) inside the
backward, which only arises when tanh is re-evaluated from x. dalpha is
formed from x, never as dx / alpha, so alpha = +inf cannot turn it into NaN.

Every step is evaluated in float64 on the stored input values (bfloat16 and
float32 inputs promote to float64 exactly; alpha * x is exact in float64
because a 24-bit by 24-bit product fits in 53 bits). sech^2 is computed as
1 / cosh(u)^2, which is free of the cancellation of 1 - tanh^2 for large
|u|; when cosh overflows the result is 0, the correct limit. IEEE special
values propagate as the arithmetic dictates: alpha = +inf with x != 0 gives
tanh = +-1, s = 0 and therefore dx = NaN (dy * gamma * inf * 0) at every
element and dalpha terms of 0; a real x = 0 with alpha = +inf gives
u = inf * 0 = NaN, which then propagates (the hazard the "Padding" bullet
describes for padded lanes; padded lanes are not part of the problem and
never enter this oracle).

Residual add fused in front of the layer (the pre-norm block pattern; a
fusion of two neighbouring steps, not something the DyT pull request
describes): for a residual stream x and a branch output r of the same shape

    h = x + r            (rounded once to the storage dtype of x)
    y = DyT(h)           (from h as stored)

and, with dres the gradient reaching h through the residual stream,

    dh = dres + dx(h, dy)     (the gradient of both x and r)

with dgamma, dbeta, dalpha those of the layer at input h. The sum x + r is
formed in float64 and rounded once (round to nearest even): for float32,
bfloat16 and float16 inputs this is the correctly rounded sum in that dtype.

Sums are taken with numpy's pairwise float64 summation over row chunks.
The oracle returns unrounded float64 results and, for the tolerance
checks, the per-element condition scale of y (|gamma t| + |beta|) and the
root-sum-of-squares (RSS) of every reduced output's terms.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .compare import rne as _rne

__all__ = [
    "forward", "backward", "forward_core", "backward_core",
    "forward_at", "backward_dx_at", "ForwardResult", "BackwardResult",
    "residual_sum", "forward_residual", "backward_residual", "backward_dh_at",
]

_CHUNK_ELEMS = 1 << 22


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def forward_core(x, alpha, gamma, beta):
    """y = gamma * tanh(alpha * x) + beta, elementwise, broadcasting gamma
    and beta along the last axis. Dtype-generic: float64 for the oracle,
    complex128 for complex-step differentiation of this same function."""
    with np.errstate(invalid="ignore"):
        u = alpha * x
        t = np.tanh(u)
        return gamma * t + beta


def _sech2(u):
    with np.errstate(over="ignore"):
        c = np.cosh(u)
        return 1.0 / (c * c)


def backward_core(x, dy, alpha, gamma):
    """Per-element backward terms (no reduction).

    Returns (dx, dgamma_terms, dbeta_terms, dalpha_terms), each shaped like x.
    """
    with np.errstate(invalid="ignore"):
        u = alpha * x
        t = np.tanh(u)
        s = _sech2(u)
        dx = dy * gamma * alpha * s
        dgamma_terms = dy * t
        dalpha_terms = dy * gamma * x * s
    dbeta_terms = dy
    return dx, dgamma_terms, dbeta_terms, dalpha_terms


@dataclass
class ForwardResult:
    y: np.ndarray        # float64, unrounded
    scale: np.ndarray    # |gamma * t| + |beta|, the condition scale of y


@dataclass
class BackwardResult:
    dx: np.ndarray       # float64 (M, N), unrounded (None if not requested)
    dgamma: np.ndarray   # float64 (N,)
    dbeta: np.ndarray    # float64 (N,)
    dalpha: float        # float64 scalar
    rss_dgamma: np.ndarray
    rss_dbeta: np.ndarray
    rss_dalpha: float


def _row_chunks(M: int, N: int):
    rows = max(1, _CHUNK_ELEMS // max(N, 1))
    for r0 in range(0, M, rows):
        yield r0, min(M, r0 + rows)


def forward(x, alpha, gamma, beta) -> ForwardResult:
    """fp64 forward over a full (M, N) input, processed in row chunks."""
    x = np.asarray(x)
    M, N = x.shape
    a = float(_f64(alpha).reshape(-1)[0])
    g = _f64(gamma).reshape(N)
    b = _f64(beta).reshape(N)
    y = np.empty((M, N), dtype=np.float64)
    scale = np.empty((M, N), dtype=np.float64)
    for r0, r1 in _row_chunks(M, N):
        xc = _f64(x[r0:r1])
        y[r0:r1] = forward_core(xc, a, g, b)
        # condition scale |gamma * t| + |beta|: the same forward with beta = 0
        scale[r0:r1] = np.abs(forward_core(xc, a, g, 0.0)) + np.abs(b)
    return ForwardResult(y, scale)


def backward(x, dy, alpha, gamma, want_dx: bool = True) -> BackwardResult:
    """fp64 backward over a full (M, N) input, processed in row chunks.

    With want_dx=False only the reductions are kept (dx is None), which
    bounds memory on large inputs."""
    x = np.asarray(x)
    M, N = x.shape
    a = float(_f64(alpha).reshape(-1)[0])
    g = _f64(gamma).reshape(N)
    dx = np.empty((M, N), dtype=np.float64) if want_dx else None
    dgamma = np.zeros(N)
    dbeta = np.zeros(N)
    dalpha = 0.0
    sq_g = np.zeros(N)
    sq_b = np.zeros(N)
    sq_a = 0.0
    for r0, r1 in _row_chunks(M, N):
        xc = _f64(x[r0:r1])
        dyc = _f64(dy[r0:r1])
        dxc, tg, tb, ta = backward_core(xc, dyc, a, g)
        if want_dx:
            dx[r0:r1] = dxc
        dgamma += tg.sum(axis=0)
        dbeta += tb.sum(axis=0)
        dalpha += float(ta.sum())
        with np.errstate(invalid="ignore", over="ignore"):
            sq_g += (tg * tg).sum(axis=0)
            sq_b += (tb * tb).sum(axis=0)
            sq_a += float((ta * ta).sum())
    return BackwardResult(dx, dgamma, dbeta, dalpha,
                          np.sqrt(sq_g), np.sqrt(sq_b), float(np.sqrt(sq_a)))


def forward_at(x_vals, cols, alpha, gamma, beta):
    """y at sampled elements, one by one: x_vals[k] sits in column cols[k].

    Returns (y, scale) as float64 arrays."""
    xv = _f64(x_vals)
    a = float(_f64(alpha).reshape(-1)[0])
    g = _f64(gamma)[cols]
    b = _f64(beta)[cols]
    return forward_core(xv, a, g, b), np.abs(forward_core(xv, a, g, 0.0)) + np.abs(b)


def backward_dx_at(x_vals, dy_vals, cols, alpha, gamma):
    """dx at sampled elements, one by one (float64)."""
    a = float(_f64(alpha).reshape(-1)[0])
    g = _f64(gamma)[cols]
    dx, _, _, _ = backward_core(_f64(x_vals), _f64(dy_vals), a, g)
    return dx


# ----------------------------------------------------------- residual add

def residual_sum(x, r, x_dtype: str) -> np.ndarray:
    """h = x + r, formed in float64 and rounded once to x_dtype (RNE)."""
    return _rne(_f64(x) + _f64(r), x_dtype)


def forward_residual(x, r, alpha, gamma, beta, x_dtype: str):
    """Residual add, then the layer on h as stored: returns (h, ForwardResult of h)."""
    h = residual_sum(x, r, x_dtype)
    return h, forward(h, alpha, gamma, beta)


def backward_residual(h, dy, dres, alpha, gamma, want_dh: bool = True):
    """Gradient of the residual-fused layer: returns (dh, BackwardResult of the
    layer at input h), dh = dres + dx in float64 (None unless want_dh), and
    the scale |dres| + |dx| of dh."""
    res = backward(h, dy, alpha, gamma, want_dx=want_dh)
    if not want_dh:
        return None, res, None
    d = _f64(dres)
    return d + res.dx, res, np.abs(d) + np.abs(res.dx)


def backward_dh_at(h_vals, dy_vals, dres_vals, cols, alpha, gamma):
    """dh at sampled elements, one by one: returns (dh, scale |dres| + |dx|)."""
    dx = backward_dx_at(h_vals, dy_vals, cols, alpha, gamma)
    d = _f64(dres_vals)
    return d + dx, np.abs(d) + np.abs(dx)
