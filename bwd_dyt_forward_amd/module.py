"""PyTorch autograd function and module for the DyT layer over the C ABI.

``DyT(num_features)`` is a drop-in layer computing
``y = weight * tanh(alpha * x) + bias`` over the last dimension of x, with
scalar ``alpha`` and per-feature ``weight`` (gamma) and ``bias`` (beta), as
the Liger-Kernel pull request "fix(dyt): use a 1D grid and tile small-width
rows" treats it (Summary: y keeps x's dtype, the parameter gradients come
back in the parameters' dtype). Forward and backward run in the HIP library;
this module only reshapes to [M, N] and wires autograd.
"""
from __future__ import annotations

import torch
from torch import nn

from . import _lib


def _rows(t: torch.Tensor) -> torch.Tensor:
    """[..., N] -> [M, N] with unit column stride and a row pitch >= N: a view
    when the leading dimensions flatten into one row stride (contiguous
    tensors, or rows sliced out of a wider buffer), else a contiguous copy."""
    n = t.shape[-1]
    if t.dim() >= 1 and (n <= 1 or t.stride(-1) == 1):
        try:
            v = t.view(-1, n)
        except RuntimeError:
            v = None
        if v is not None and (v.size(0) <= 1 or v.stride(0) >= n) and (n <= 1 or v.stride(1) == 1):
            return v
    return t.contiguous().view(-1, n)


def _dense_rows(t: torch.Tensor) -> torch.Tensor:
    """[..., N] -> contiguous [M, N] (the residual-fused calls take dense rows)."""
    t = t.contiguous()
    return t.view(-1, t.shape[-1])


class DyTFunction(torch.autograd.Function):
    """Autograd wrapper: forward saves x (the backward recomputes tanh from x)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, alpha: torch.Tensor, gamma: torch.Tensor,
                beta: torch.Tensor) -> torch.Tensor:
        x2 = _rows(x)
        y = _lib.dyt_forward(x2, alpha, gamma, beta)
        ctx.save_for_backward(x2, alpha, gamma)
        ctx.x_shape = x.shape
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x2, alpha, gamma = ctx.saved_tensors
        dy2 = _rows(dy.to(x2.dtype))
        dx, dalpha, dgamma, dbeta = _lib.dyt_backward(x2, dy2, alpha, gamma)
        return dx.view(ctx.x_shape), dalpha, dgamma, dbeta


def dyt(x: torch.Tensor, alpha: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor) -> torch.Tensor:
    """Functional form with autograd support."""
    return DyTFunction.apply(x, alpha, gamma, beta)


class DyT(nn.Module):
    """Dynamic Tanh layer: ``weight * tanh(alpha * x) + bias`` over the last dim.

    ``alpha_init`` defaults to 0.5; ``weight`` starts at 1 and ``bias`` at 0.
    Parameters live in ``dtype`` (float32, bfloat16 or float16); inputs may be
    any of the three independently of it.
    """

    def __init__(self, num_features: int, alpha_init: float = 0.5, dtype=torch.float32,
                 device=None):
        super().__init__()
        kw = {"dtype": dtype, "device": device}
        self.num_features = num_features
        self.alpha = nn.Parameter(torch.full((1,), float(alpha_init), **kw))
        self.weight = nn.Parameter(torch.ones(num_features, **kw))
        self.bias = nn.Parameter(torch.zeros(num_features, **kw))

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.num_features:
            raise ValueError(f"expected last dimension {self.num_features}, got {x.shape[-1]}")
        return DyTFunction.apply(x, self.alpha, self.weight, self.bias)

    def extra_repr(self) -> str:
        return f"{self.num_features}, alpha={float(self.alpha.detach().float().cpu()[0]):.4g}"


class DyTResidualFunction(torch.autograd.Function):
    """Autograd wrapper of the residual-fused layer: (x, r) -> (h = x + r, y = DyT(h)).

    The backward receives the gradients of both outputs and returns
    dh = grad_h + DyT-backward(grad_y) for x and for r (one fused kernel when
    both are present).
    """

    @staticmethod
    def forward(ctx, x: torch.Tensor, r: torch.Tensor, alpha: torch.Tensor, gamma: torch.Tensor,
                beta: torch.Tensor):
        x2 = _dense_rows(x)
        r2 = _dense_rows(r.to(x.dtype))
        h, y = _lib.dyt_forward_residual(x2, r2, alpha, gamma, beta)
        ctx.save_for_backward(h, alpha, gamma)
        ctx.set_materialize_grads(False)   # an unused output's gradient arrives as None
        ctx.x_shape = x.shape
        return h.view(x.shape), y.view(x.shape)

    @staticmethod
    def backward(ctx, grad_h: torch.Tensor | None, grad_y: torch.Tensor | None):
        h, alpha, gamma = ctx.saved_tensors
        shape = ctx.x_shape
        if grad_y is None:
            dh = _dense_rows(grad_h.to(h.dtype)).view(shape)
            return dh, dh, None, None, None
        dy2 = _dense_rows(grad_y.to(h.dtype))
        if grad_h is None:
            dh, dalpha, dgamma, dbeta = _lib.dyt_backward(h, dy2, alpha, gamma)
        else:
            dres = _dense_rows(grad_h.to(h.dtype))
            dh, dalpha, dgamma, dbeta = _lib.dyt_backward_residual(h, dy2, dres, alpha, gamma)
        # One tensor object for both inputs (as torch's own add backward does):
        # two views would be two tensors on one storage, which gradient
        # accumulation into leaf x and r would then both adopt, aliasing
        # x.grad with r.grad. With one object it copies before it keeps one.
        dh = dh.view(shape)
        return dh, dh, dalpha, dgamma, dbeta


def dyt_residual(x: torch.Tensor, r: torch.Tensor, alpha: torch.Tensor, gamma: torch.Tensor,
                 beta: torch.Tensor):
    """(h, y) = (x + r, DyT(x + r)) with autograd support."""
    return DyTResidualFunction.apply(x, r, alpha, gamma, beta)


class DyTResidual(DyT):
    """DyT with the residual add fused in front: ``forward(x, r)`` returns
    ``(h, y)`` with ``h = x + r`` (the new residual stream, in x's dtype) and
    ``y = weight * tanh(alpha * h) + bias``."""

    def forward(self, x: torch.Tensor, r: torch.Tensor):  # type: ignore[override]
        if x.shape[-1] != self.num_features or r.shape != x.shape:
            raise ValueError(f"expected x and r of equal shape with last dimension {self.num_features}")
        return DyTResidualFunction.apply(x, r, self.alpha, self.weight, self.bias)
