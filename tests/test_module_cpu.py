"""Host logic of the binding and the autograd layer, on the CPU.

The library's kernels need a GPU, so the autograd wiring is exercised here
with the two library calls replaced by plain torch stand-ins on CPU
tensors (test scaffolding only: the package has no CPU path). What is
checked is the wiring itself: which gradient goes to which input, and that
gradients accumulated into leaf tensors over several backward passes do not
share storage."""
import pytest
import torch

import bwd_dyt_forward_amd as dyt
from bwd_dyt_forward_amd import _lib, module


def _fake_forward_residual(x, r, alpha, gamma, beta):
    h = x + r
    return h, gamma * torch.tanh(alpha * h) + beta


def _fake_backward_residual(h, dy, dres, alpha, gamma):
    t = torch.tanh(alpha * h)
    g = dy * gamma * (1 - t * t)
    return dres + g * alpha, (g * h).sum().reshape(1), (dy * t).sum(0), dy.sum(0)


def _fake_backward(h, dy, alpha, gamma):
    return _fake_backward_residual(h, dy, torch.zeros_like(h), alpha, gamma)


@pytest.fixture
def cpu_kernels(monkeypatch):
    monkeypatch.setattr(_lib, "dyt_forward_residual", _fake_forward_residual)
    monkeypatch.setattr(_lib, "dyt_backward_residual", _fake_backward_residual)
    monkeypatch.setattr(_lib, "dyt_backward", _fake_backward)


@pytest.mark.parametrize("use_h", [True, False])
def test_residual_grads_of_leaf_inputs_accumulate_separately(cpu_kernels, use_h):
    g = torch.Generator().manual_seed(5)
    x = torch.randn(6, 8, generator=g, requires_grad=True)
    r = torch.randn(6, 8, generator=g, requires_grad=True)
    a = torch.tensor([0.7], requires_grad=True)
    gm = torch.randn(8, generator=g, requires_grad=True)
    bt = torch.randn(8, generator=g, requires_grad=True)

    def loss():
        h, y = module.dyt_residual(x, r, a, gm, bt)
        return (y * y).sum() + ((h * 3).sum() if use_h else 0)

    loss().backward()
    gx, gr = x.grad.clone(), r.grad.clone()
    assert torch.equal(gx, gr)
    assert x.grad.data_ptr() != r.grad.data_ptr()
    loss().backward()
    assert torch.equal(x.grad, 2 * gx)
    assert torch.equal(r.grad, 2 * gr)
    assert x.grad.data_ptr() != r.grad.data_ptr()


def test_residual_grad_of_h_alone(cpu_kernels):
    x = torch.randn(3, 4, requires_grad=True)
    r = torch.randn(3, 4, requires_grad=True)
    a, gm, bt = torch.tensor([0.5]), torch.ones(4), torch.zeros(4)
    for _ in range(2):
        h, _y = module.dyt_residual(x, r, a, gm, bt)
        (2 * h).sum().backward()
    assert torch.equal(x.grad, torch.full((3, 4), 4.0))
    assert torch.equal(r.grad, torch.full((3, 4), 4.0))
    assert x.grad.data_ptr() != r.grad.data_ptr()


def test_check_params_rejects_host_and_foreign_tensors():
    dev = torch.device("cuda", 0)
    a, v = torch.tensor([0.5]), torch.ones(4)
    with pytest.raises(ValueError, match="alpha"):
        _lib._check_params(4, dev, a, v, v)
    with pytest.raises(ValueError):
        _lib._check_params(4, dev, a.numpy(), v, v)
    # the device check comes first: a host alpha never reaches a size check
    with pytest.raises(ValueError, match="alpha must be a tensor on"):
        _lib._check_params(4, dev, torch.ones(3), v)


def test_activation_on_host_is_rejected_before_any_call():
    x = torch.ones(4, 8)
    p = torch.ones(8)
    for call in (lambda: dyt.dyt_forward(x, p[:1], p, p),
                 lambda: dyt.dyt_backward(x, x, p[:1], p),
                 lambda: dyt.dyt_forward_residual(x, x, p[:1], p, p),
                 lambda: dyt.dyt_backward_residual(x, x, x, p[:1], p)):
        with pytest.raises(ValueError):
            call()
