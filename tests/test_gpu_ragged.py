"""Awkward row widths. Rows whose length is not a multiple of the 16-byte
vector width (and rows wider than a tile): the vector kernels shift each
row's last vector back to end at the row's end, so its first elements
rewrite bytes a neighbouring slot owns (or, when the last column block is
shorter than a vector, bytes of the previous block). Widths that fill the
default tiles poorly run re-tiled plans (K = 3 or 4 slots, packed tiles of
up to 8,192 elements). Checked here: every output against the oracle, guard
canaries around every output, unaligned bases equal to aligned ones bit for
bit, row-strided launches equal to contiguous ones bit for bit (with the
element-wise kernels: y and dx, the gradients equal to a second strided
launch), and the residual-fused layer."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import TORCH_DT, assert_reports, full_reports, log
from oracle import compare, dyt_oracle

pytestmark = pytest.mark.gpu

CANARY = -12288.0                     # exact in every x dtype


@pytest.fixture(scope="module")
def dyt():
    import __graft_entry__ as ge
    ge._ensure_built()
    import bwd_dyt_forward_amd as m
    return m


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy().copy()


def _embedded(t: torch.Tensor, before: int, after: int, fill=CANARY):
    n = t.numel()
    buf = torch.full((before + n + after,), fill, dtype=t.dtype, device=t.device)
    v = buf[before:before + n].view(t.shape)
    v.copy_(t)
    return v, buf


# (M, N, x dtype, param dtype): one column block, or several with a ragged
# last one
SHAPES = [
    (257, 4095, "bf16", "f32"),
    (33, 10001, "bf16", "bf16"),
    (129, 2051, "f32", "f32"),
    (65, 3001, "f16", "f32"),
    (40, 4097, "f32", "f32"),
    (9, 20003, "bf16", "f32"),
]
# last column block shorter than one vector (1 or 2 columns); the CPU test
# test_short_last_block_shapes checks that the plan still makes them so
SHORT_LAST = [(3, 261121, "f32", "f32"), (3, 522241, "bf16", "f32"), (2, 522242, "f16", "bf16")]


def _inputs(M, N, xdt, pdt, seed):
    return workloads.custom(M, N, xdt, pdt, alpha=0.8, seed=seed)


def _upload(inp, xdt, pdt):
    xt, pt = TORCH_DT[xdt], TORCH_DT[pdt]
    t = lambda a, dt: torch.from_numpy(a).to("cuda").to(dt)
    return (t(inp.x, xt), t(inp.dy, xt), t(inp.alpha, pt), t(inp.gamma, pt), t(inp.beta, pt))


def _check_shape(dyt, M, N, xdt, pdt):
    log(f"[ragged] M={M} N={N} x={xdt} p={pdt}")
    inp = _inputs(M, N, xdt, pdt, seed=N)
    x, dy, a, g, b = _upload(inp, xdt, pdt)
    pad = 64
    y, ybuf = _embedded(torch.empty_like(x), pad, pad)
    dx, dxbuf = _embedded(torch.empty_like(x), pad, pad)
    dyt.dyt_forward(x, a, g, b, y=y)
    _, da, dg, db = dyt.dyt_backward(x, dy, a, g, dx=dx)
    torch.cuda.synchronize()
    for buf in (ybuf, dxbuf):
        assert bool((buf[:pad] == CANARY).all()) and bool((buf[-pad:] == CANARY).all())
    assert_reports(f"ragged {M}x{N}", full_reports(inp, y, dx, da, dg, db))
    # unaligned bases: same kernels, same bits
    xu, _ = _embedded(x, 1, 0)
    dyu, _ = _embedded(dy, 1, 0)
    yu, _ = _embedded(torch.empty_like(x), 1, 0)
    dxu, _ = _embedded(torch.empty_like(x), 1, 0)
    assert xu.data_ptr() % 16 != 0
    dyt.dyt_forward(xu, a, g, b, y=yu)
    _, dau, dgu, dbu = dyt.dyt_backward(xu, dyu, a, g, dx=dxu)
    # row-strided: same tiles, gaps untouched; packed rows whose length is
    # not a multiple of the vector width take the element-wise kernels
    def strided(ld):
        xs = torch.full((M, ld), CANARY, dtype=x.dtype, device="cuda")[:, :N]
        xs.copy_(x)
        dys = torch.full((M, ld + 1), CANARY, dtype=x.dtype, device="cuda")[:, :N]
        dys.copy_(dy)
        ysb = torch.full((M, ld + 5), CANARY, dtype=x.dtype, device="cuda")
        dxsb = torch.full((M, ld + 2), CANARY, dtype=x.dtype, device="cuda")
        ys, dxs = ysb[:, :N], dxsb[:, :N]
        dyt.dyt_forward(xs, a, g, b, y=ys)
        _, das, dgs, dbs = dyt.dyt_backward(xs, dys, a, g, dx=dxs)
        return ys, dxs, das, dgs, dbs, ysb, dxsb
    ys, dxs, das, dgs, dbs, ysb, dxsb = strided(N + 3)
    torch.cuda.synchronize()
    v = 16 // x.element_size()
    elementwise = bool(dyt.dyt_get_plan(M, N, xdt, pdt)["packed"]) and N % v != 0
    if elementwise:
        grads = strided(N + 9)[2:5]
        torch.cuda.synchronize()
    else:
        grads = (da, dg, db)
    for u, w in ((yu, y), (dxu, dx), (dau, da), (dgu, dg), (dbu, db), (ys, y), (dxs, dx),
                 (das, grads[0]), (dgs, grads[1]), (dbs, grads[2])):
        assert np.array_equal(_bits(u), _bits(w))
    assert bool((ysb[:, N:] == CANARY).all()) and bool((dxsb[:, N:] == CANARY).all())
    if elementwise:
        assert_reports(f"ragged strided {M}x{N}", full_reports(inp, ys, dxs, das, dgs, dbs))


@pytest.mark.parametrize("M,N,xdt,pdt", SHAPES)
def test_ragged_rows(dyt, M, N, xdt, pdt):
    _check_shape(dyt, M, N, xdt, pdt)


# re-tiled for slot occupancy (the CPU test test_occupancy_retiling checks
# that these shapes get K = 3 / 4 and packed tiles beyond 4,096 elements)
RETILED = [(2800, 1500, "bf16", "f32"), (1100, 5120, "bf16", "f32"), (2000, 2560, "bf16", "bf16"),
           (1700, 2560, "f32", "f32"), (2100, 4104, "f32", "f32"), (1400, 3072, "bf16", "f32")]


@pytest.mark.parametrize("M,N,xdt,pdt", RETILED)
def test_retiled_widths(dyt, M, N, xdt, pdt):
    _check_shape(dyt, M, N, xdt, pdt)


@pytest.mark.parametrize("M,N,xdt,pdt", SHORT_LAST)
def test_short_last_block(dyt, M, N, xdt, pdt):
    """Last column block shorter than one vector: its one vector reaches back
    into the previous block of the same row."""
    _check_shape(dyt, M, N, xdt, pdt)


@pytest.mark.parametrize("M,N,xdt", [(65, 4095, "bf16"), (17, 10001, "f32")])
def test_ragged_residual(dyt, M, N, xdt):
    """The residual-fused layer on ragged rows: h bit for bit, y, dh and the
    gradients within tolerance."""
    log(f"[ragged residual] M={M} N={N} x={xdt}")
    inp = _inputs(M, N, xdt, "f32", seed=7 * N)
    r, dres = workloads.residual_pair(M, N, xdt, 3)
    x, dy, a, g, b = _upload(inp, xdt, "f32")
    xt = TORCH_DT[xdt]
    rt = torch.from_numpy(r).to("cuda").to(xt)
    drt = torch.from_numpy(dres).to("cuda").to(xt)
    h, y = dyt.dyt_forward_residual(x, rt, a, g, b)
    dh, da, dg, db = dyt.dyt_backward_residual(h, dy, drt, a, g)
    torch.cuda.synchronize()
    h_ref, f = dyt_oracle.forward_residual(inp.x, r, inp.alpha, inp.gamma, inp.beta, xdt)
    dh_ref, bw, scale = dyt_oracle.backward_residual(h_ref, inp.dy, dres, inp.alpha, inp.gamma)
    npf = lambda v: v.float().cpu().numpy()
    reps = [compare.check_exact(npf(h), h_ref, "h"),
            compare.check_y(npf(y), f.y, f.scale, xdt),
            compare.check_dh(npf(dh), dh_ref, scale, xdt),
            compare.check_grad(npf(dg), bw.dgamma, bw.rss_dgamma, "f32", "dgamma"),
            compare.check_grad(npf(db), bw.dbeta, bw.rss_dbeta, "f32", "dbeta"),
            compare.check_grad(npf(da), bw.dalpha, bw.rss_dalpha, "f32", "dalpha")]
    assert_reports(f"ragged residual {M}x{N}", reps)
