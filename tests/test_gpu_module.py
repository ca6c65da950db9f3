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
@pytest.mark.parametrize("alpha0", [0.7, -0.9])
def test_module_forward_backward_matches_oracle(dyt, xdt, pdt, shape, alpha0):
    log(f"[module] shape={shape} x={xdt} p={pdt} alpha={alpha0}")
    g = torch.Generator().manual_seed(sum(shape))
    N = shape[-1]
    x32 = torch.randn(shape, generator=g) * 1.5
    dy32 = torch.randn(shape, generator=g)
    xd, pd = TORCH_DT[xdt], TORCH_DT[pdt]
    layer = dyt.DyT(N, alpha_init=alpha0, dtype=pd, device="cuda")
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
    assert_reports(f"module {shape} {xdt}/{pdt} alpha {alpha0}", [
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


def test_residual_module_leaf_grads_accumulate_separately(dyt):
    """x and r both leaves: each gets dh, in its own storage, and a second
    backward pass doubles both (no aliasing between x.grad and r.grad)."""
    layer = dyt.DyTResidual(64, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn(32, 64, device="cuda", generator=g).requires_grad_(True)
    r = torch.randn(32, 64, device="cuda", generator=g).requires_grad_(True)

    def loss():
        h, y = layer(x, r)
        return (y * y).sum() + 3 * h.sum()

    loss().backward()
    gx, gr = x.grad.clone(), r.grad.clone()
    assert torch.equal(gx, gr) and x.grad.data_ptr() != r.grad.data_ptr()
    loss().backward()
    assert torch.equal(x.grad, 2 * gx) and torch.equal(r.grad, 2 * gr)
    assert x.grad.data_ptr() != r.grad.data_ptr()


def test_host_parameters_are_rejected_before_launch(dyt):
    x = torch.randn(8, 16, device="cuda")
    a, gm, bt = torch.tensor([0.5]), torch.ones(16), torch.zeros(16)
    with pytest.raises(ValueError):
        dyt.dyt_forward(x, a, gm.cuda(), bt.cuda())
    with pytest.raises(ValueError):
        dyt.dyt_forward(x, a.cuda(), gm, bt.cuda())
    with pytest.raises(ValueError):
        dyt.dyt_backward(x, x, a, gm.cuda())
    with pytest.raises(ValueError):
        dyt.dyt_forward_residual(x, x, a.cuda(), gm.cuda(), bt)


def test_explicit_side_stream_matches_current_stream(dyt):
    x = torch.randn(1000, 96, device="cuda")
    dy = torch.randn(1000, 96, device="cuda")
    a = torch.tensor([0.7], device="cuda")
    gm, bt = torch.randn(96, device="cuda"), torch.randn(96, device="cuda")
    y0 = dyt.dyt_forward(x, a, gm, bt)
    b0 = dyt.dyt_backward(x, dy, a, gm)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for stream in (s, s.cuda_stream):
        y1 = dyt.dyt_forward(x, a, gm, bt, stream=stream)
        b1 = dyt.dyt_backward(x, dy, a, gm, stream=stream)
        s.synchronize()
        assert torch.equal(y0, y1)
        for u, v in zip(b0, b1):
            assert torch.equal(u, v)
