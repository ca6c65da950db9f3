"""The autograd drop-in (DyT module / DyTFunction) against the fp64 oracle."""
import numpy as np
import pytest
import torch

from gpu_util import TORCH_DT, assert_reports, log
from oracle import compare, dyt_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dyt():
    import __graft_entry__ as ge
    ge._ensure_built()
    import bwd_dyt_forward_amd as m
    return m


@pytest.mark.parametrize("xdt,pdt", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"), ("f16", "f16")])
@pytest.mark.parametrize("shape", [(4, 129, 64), (3, 5, 4096), (1000, 17)])
def test_module_forward_backward_matches_oracle(dyt, xdt, pdt, shape):
    log(f"[module] shape={shape} x={xdt} p={pdt}")
    g = torch.Generator().manual_seed(sum(shape))
    N = shape[-1]
    x32 = torch.randn(shape, generator=g) * 1.5
    dy32 = torch.randn(shape, generator=g)
    xd, pd = TORCH_DT[xdt], TORCH_DT[pdt]
    layer = dyt.DyT(N, alpha_init=0.7, dtype=pd, device="cuda")
    with torch.no_grad():
        layer.weight.copy_((1 + 0.1 * torch.randn(N, generator=g)).to(pd))
        layer.bias.copy_((0.1 * torch.randn(N, generator=g)).to(pd))
    x = x32.to(xd).cuda().requires_grad_(True)
    dy = dy32.to(xd).cuda()
    y = layer(x)
    assert y.dtype == xd and y.shape == x.shape
    y.backward(dy)
    assert x.grad.dtype == xd and layer.alpha.grad.dtype == pd and layer.weight.grad.dtype == pd
    xs = x.detach().float().cpu().numpy().reshape(-1, N)
    dys = dy.float().cpu().numpy().reshape(-1, N)
    a = layer.alpha.detach().float().cpu().numpy()
    gm = layer.weight.detach().float().cpu().numpy()
    bt = layer.bias.detach().float().cpu().numpy()
    f = dyt_oracle.forward(xs, a, gm, bt)
    r = dyt_oracle.backward(xs, dys, a, gm)
    t = lambda v: v.detach().float().cpu().numpy().astype(np.float64)
    assert_reports(f"module {shape} {xdt}/{pdt}", [
        compare.check_y(t(y).reshape(-1, N), f.y, f.scale, xdt),
        compare.check_dx(t(x.grad).reshape(-1, N), r.dx, xdt),
        compare.check_grad(t(layer.weight.grad), r.dgamma, r.rss_dgamma, pdt, "dgamma"),
        compare.check_grad(t(layer.bias.grad), r.dbeta, r.rss_dbeta, pdt, "dbeta"),
        compare.check_grad(t(layer.alpha.grad), r.dalpha, r.rss_dalpha, pdt, "dalpha"),
    ])


def test_module_gradient_accumulates_like_autograd(dyt):
    """Two backward passes accumulate parameter gradients (autograd semantics)."""
    layer = dyt.DyT(64, device="cuda")
    x = torch.randn(32, 64, device="cuda")
    layer(x).sum().backward()
    g1 = layer.weight.grad.clone()
    layer(x).sum().backward()
    assert torch.equal(layer.weight.grad, 2 * g1)


def test_module_rejects_wrong_width(dyt):
    layer = dyt.DyT(8, device="cuda")
    with pytest.raises(ValueError):
        layer(torch.randn(2, 9, device="cuda"))
