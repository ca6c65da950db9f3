"""Row-strided activations (dyt_forward_strided / dyt_backward_strided):
results equal the contiguous calls bit for bit (same tiling, same partial
rows), on both tile layouts and with pitches of any alignment; packed rows
whose length is not a multiple of the vector width take the element-wise
kernels. The gaps between rows are never written."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import TORCH_DT, assert_reports, full_reports, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dyt():
    import __graft_entry__ as ge
    ge._ensure_built()
    import bwd_dyt_forward_amd as m
    return m


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy().copy()


CANARY = -12288.0


def _strided(src: torch.Tensor, pad: int, fill=CANARY) -> torch.Tensor:
    """src copied into an [M, N + pad] buffer filled with a canary; returns the
    [M, N] view (row pitch N + pad)."""
    M, N = src.shape
    buf = torch.full((M, N + pad), fill, dtype=src.dtype, device=src.device)
    v = buf[:, :N]
    v.copy_(src)
    return v


SHAPES = [  # (M, N, x dtype, param dtype, pads for x / dy / outputs)
    (2049, 32, "bf16", "f32", (8, 16, 24)),        # packed, vector kernels
    (1031, 17, "f32", "f32", (3, 1, 7)),           # packed, element-wise (N % V != 0)
    (333, 100, "f16", "f16", (4, 12, 28)),         # packed, element-wise (N % V != 0)
    (301, 64, "bf16", "bf16", (1, 8, 8)),          # packed, odd pitch: vector kernels
    (65, 4096, "bf16", "f32", (64, 8, 128)),       # row segments
    (9, 20000, "f32", "f32", (4, 0, 12)),          # row segments, several column blocks
    (7, 5000, "f32", "bf16", (1, 2, 3)),           # row segments, odd pitches
    (11, 4099, "bf16", "f32", (5, 1, 2)),          # row segments, N % V != 0
]


def _vector_kernels(N: int, sx: int, packed: bool) -> bool:
    """The documented rule: every pitch takes the 16-byte kernels except
    packed rows whose length is not a multiple of the vector width."""
    return not packed or N % (16 // sx) == 0


def _strided_run(dyt, x, dy, a, g, b, pads):
    px, pd, po = pads
    pdx = po + 8 if po else 0
    xs, dys = _strided(x, px), _strided(dy, pd)
    ys = _strided(torch.zeros_like(x), po)
    dxs = _strided(torch.zeros_like(x), pdx)
    dyt.dyt_forward(xs, a, g, b, y=ys)
    _, da, dg, db = dyt.dyt_backward(xs, dys, a, g, dx=dxs)
    return ys, dxs, da, dg, db, po, pdx


@pytest.mark.parametrize("M,N,xdt,pdt,pads", SHAPES)
def test_strided_equals_contiguous(dyt, M, N, xdt, pdt, pads):
    """Same tiling as the contiguous call. With the vector kernels every
    output is the contiguous call's bit for bit; with the element-wise ones
    (packed rows, N not a multiple of the vector width) y and dx are, the
    gradients match another strided launch bit for bit and the oracle."""
    log(f"[strided] M={M} N={N} x={xdt} p={pdt} pads={pads}")
    inp = workloads.custom(M, N, xdt, pdt, alpha=0.7, seed=M * 31 + N)
    xt, pt = TORCH_DT[xdt], TORCH_DT[pdt]
    sx = torch.tensor([], dtype=xt).element_size()
    dev = "cuda"
    x = torch.from_numpy(inp.x).to(dev).to(xt)
    dy = torch.from_numpy(inp.dy).to(dev).to(xt)
    a = torch.from_numpy(inp.alpha).to(dev).to(pt)
    g = torch.from_numpy(inp.gamma).to(dev).to(pt)
    b = torch.from_numpy(inp.beta).to(dev).to(pt)
    packed = bool(dyt.dyt_get_plan(M, N, xdt, pdt)["packed"])
    assert packed == bool(dyt.dyt_get_forward_plan(M, N, xdt, pdt)["packed"])
    vec = _vector_kernels(N, sx, packed)
    y0 = dyt.dyt_forward(x, a, g, b)
    dx0, da0, dg0, db0 = dyt.dyt_backward(x, dy, a, g)
    ys, dxs, da, dg, db, po, pdx = _strided_run(dyt, x, dy, a, g, b, pads)
    torch.cuda.synchronize()
    log(f"[strided] vector kernels: {vec}")
    assert np.array_equal(_bits(ys), _bits(y0))
    assert np.array_equal(_bits(dxs), _bits(dx0))
    if vec:
        refs = (da0, dg0, db0)
    else:
        _, _, *refs, _, _ = _strided_run(dyt, x, dy, a, g, b, tuple(q + 5 for q in pads))
        torch.cuda.synchronize()
    for u, v in zip((da, dg, db), refs):
        assert np.array_equal(_bits(u), _bits(v))
    # the gaps between rows are untouched
    for out, pad in ((ys, po), (dxs, pdx)):
        if pad:
            gap = out.as_strided((M, pad), (N + pad, 1), out.storage_offset() + N)
            assert bool((gap == CANARY).all())
    # and the results are right (oracle)
    assert_reports(f"strided {M}x{N}", full_reports(inp, ys, dxs, da, dg, db))


def test_strided_module_autograd(dyt):
    """The autograd layer takes rows sliced out of a wider buffer ([B, S, N]
    view with row pitch 2N) as they are; values and gradients equal those of
    a contiguous copy bit for bit."""
    B, S, N = 3, 171, 48
    torch.manual_seed(5)
    big = torch.randn(B, S, 2 * N, device="cuda").to(torch.bfloat16)
    layer = dyt.DyT(N, alpha_init=0.6, device="cuda")
    with torch.no_grad():
        layer.weight.normal_(1.0, 0.1)
        layer.bias.normal_(0.0, 0.1)
    g_out = torch.randn(B, S, N, device="cuda").to(torch.bfloat16)
    res = []
    for xin in (big[:, :, N:], big[:, :, N:].contiguous()):
        xin = xin.detach().requires_grad_(True)
        layer.zero_grad(set_to_none=True)
        y = layer(xin)
        y.backward(g_out)
        res.append((y.detach(), xin.grad, layer.alpha.grad.clone(), layer.weight.grad.clone(),
                    layer.bias.grad.clone()))
    torch.cuda.synchronize()
    for u, v in zip(*res):
        assert np.array_equal(_bits(u), _bits(v))
