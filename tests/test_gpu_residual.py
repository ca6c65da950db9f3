"""The residual-fused layer on the GPU: h = x + r (rounded once), y = DyT(h),
and its backward dh = dres + dx with the layer's parameter gradients.

Parity: h bit for bit against the oracle's rounded sum; y, dh and the
gradients within the oracle tolerances (oracle/compare.py), on fixed
shapes and on a seeded random list (widths, dtypes, alpha of either sign,
aligned or unaligned bases). Properties (bitwise): a zero branch reproduces the plain forward, a zero residual
gradient the plain backward, the split backward the single call, and
unaligned bases the aligned call."""
import math
import os

import numpy as np
import pytest
import torch

import workloads
from gpu_util import TORCH_DT, assert_reports, log, to_np
from oracle import compare, dyt_oracle

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


def _setup(M, N, xdt, pdt, alpha, seed=0, sigma=1.0):
    inp = workloads.custom(M, N, xdt, pdt, alpha=alpha, x_sigma=sigma, seed=seed)
    r, dres = workloads.residual_pair(M, N, xdt, seed)
    xt, pt = TORCH_DT[xdt], TORCH_DT[pdt]
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)
    d = dict(x=dev(inp.x, xt), r=dev(r, xt), dy=dev(inp.dy, xt), dres=dev(dres, xt),
             alpha=dev(inp.alpha, pt), gamma=dev(inp.gamma, pt), beta=dev(inp.beta, pt))
    return inp, r, dres, d


def _reports(inp, r, dres, h, y, dh, da, dg, db):
    xdt, pdt = inp.x_dtype, inp.p_dtype
    h_ref, f = dyt_oracle.forward_residual(inp.x, r, inp.alpha, inp.gamma, inp.beta, xdt)
    dh_ref, bw, scale = dyt_oracle.backward_residual(h_ref, inp.dy, dres, inp.alpha, inp.gamma)
    dga = np.abs(inp.dy.astype(np.float64) * inp.gamma.astype(np.float64) * float(inp.alpha[0]))
    return [
        compare.check_exact(to_np(h), h_ref, "h"),
        compare.check_y(to_np(y), f.y, f.scale, xdt),
        compare.check_dh(to_np(dh), dh_ref, scale, xdt, dga),
        compare.check_grad(to_np(dg), bw.dgamma, bw.rss_dgamma, pdt, "dgamma"),
        compare.check_grad(to_np(db), bw.dbeta, bw.rss_dbeta, pdt, "dbeta"),
        compare.check_grad(to_np(da), bw.dalpha, bw.rss_dalpha, pdt, "dalpha"),
    ]


SHAPES = [
    (1024, 64, "f32", "f32", 0.5),
    (65537, 16, "bf16", "f32", 0.8),
    (1003, 17, "f32", "f32", float("inf")),
    (5003, 100, "f16", "f16", 0.5),
    (301, 255, "bf16", "bf16", 1.0),
    (1031, 300, "f16", "f32", 0.7),
    (64, 4096, "bf16", "f32", 0.5),
    (33, 20000, "f32", "f32", 0.5),
    (1, 5000, "f32", "bf16", 0.5),
    (7, 3, "bf16", "f32", 0.5),
    (100003, 255, "f32", "f32", 0.5),   # packed tiles of two slots (the plain backward's plan)
]


@pytest.mark.parametrize("M,N,xdt,pdt,alpha", SHAPES)
def test_residual_parity(dyt, M, N, xdt, pdt, alpha):
    log(f"[residual parity] M={M} N={N} x={xdt} p={pdt} alpha={alpha}")
    inp, r, dres, d = _setup(M, N, xdt, pdt, alpha, seed=M + N)
    h, y = dyt.dyt_forward_residual(d["x"], d["r"], d["alpha"], d["gamma"], d["beta"])
    dh, da, dg, db = dyt.dyt_backward_residual(h, d["dy"], d["dres"], d["alpha"], d["gamma"])
    torch.cuda.synchronize()
    assert_reports(f"residual {M}x{N} {xdt}/{pdt}", _reports(inp, r, dres, h, y, dh, da, dg, db))


def _fuzz_cases(seed=int(os.environ.get("DYT_FUZZ_SEED", "20251203")),
                n=int(os.environ.get("DYT_RES_FUZZ_CASES", "24"))):
    """Random residual problems of at most 2^21 elements (every element is
    compared): N log-uniform in 1 .. 24,000, all dtype pairs, alpha in
    +-{0.3, 0.8, 1.7}, every activation and output at an aligned base or one
    element off it."""
    rng = np.random.default_rng(seed)
    out = []
    dts = ["f32", "bf16", "f16"]
    for i in range(n):
        N = int(round(math.exp(rng.uniform(0.0, math.log(24000.0)))))
        M = max(1, int(rng.integers(1 << 10, 1 << 21)) // N)
        xdt, pdt = dts[int(rng.integers(0, 3))], dts[int(rng.integers(0, 3))]
        alpha = float(rng.choice([0.3, 0.8, 1.7])) * float(rng.choice([-1.0, 1.0]))
        out.append((i, M, N, xdt, pdt, alpha, bool(rng.integers(0, 2))))
    return out


FUZZ = _fuzz_cases()


def _off_by_one(t: torch.Tensor) -> torch.Tensor:
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("case", FUZZ, ids=[f"{c[0]}-{c[1]}x{c[2]}-{c[3]}-{c[4]}" for c in FUZZ])
def test_residual_fuzz(dyt, case):
    i, M, N, xdt, pdt, alpha, unaligned = case
    log(f"[residual fuzz {i}] M={M} N={N} x={xdt} p={pdt} alpha={alpha} unaligned={unaligned}")
    inp, r, dres, d = _setup(M, N, xdt, pdt, alpha, seed=2000 + i, sigma=1.5)
    place = _off_by_one if unaligned else (lambda t: t)
    x, rr, dy, dr = (place(d[k]) for k in ("x", "r", "dy", "dres"))
    h = place(torch.zeros_like(d["x"]))
    y = place(torch.zeros_like(d["x"]))
    dh = place(torch.zeros_like(d["x"]))
    dyt.dyt_forward_residual(x, rr, d["alpha"], d["gamma"], d["beta"], h=h, y=y)
    _, da, dg, db = dyt.dyt_backward_residual(h, dy, dr, d["alpha"], d["gamma"], dh=dh)
    torch.cuda.synchronize()
    assert (h.data_ptr() % 16 != 0) == unaligned
    assert_reports(f"residual fuzz {i}", _reports(inp, r, dres, h, y, dh, da, dg, db))


@pytest.mark.parametrize("M,N,xdt", [(2049, 32, "bf16"), (40, 4096, "f16"), (501, 100, "f32")])
def test_zero_branch_and_zero_residual_gradient_are_the_plain_layer(dyt, M, N, xdt):
    """r = -0: h == x and y == dyt_forward(x); dres = -0: dh == dyt_backward's
    dx and the gradients are the plain ones, all bit for bit (x + (-0) = x
    for every x, including -0)."""
    log(f"[residual zero] M={M} N={N} x={xdt}")
    inp, r, dres, d = _setup(M, N, xdt, "f32", 0.6, seed=5)
    mz = torch.full_like(d["x"], -0.0)
    h, y = dyt.dyt_forward_residual(d["x"], mz, d["alpha"], d["gamma"], d["beta"])
    y0 = dyt.dyt_forward(d["x"], d["alpha"], d["gamma"], d["beta"])
    dh, da, dg, db = dyt.dyt_backward_residual(d["x"], d["dy"], mz, d["alpha"], d["gamma"])
    dx0, da0, dg0, db0 = dyt.dyt_backward(d["x"], d["dy"], d["alpha"], d["gamma"])
    torch.cuda.synchronize()
    assert np.array_equal(_bits(h), _bits(d["x"]))
    assert np.array_equal(_bits(y), _bits(y0))
    assert np.array_equal(_bits(dh), _bits(dx0))
    for a, b in ((da, da0), (dg, dg0), (db, db0)):
        assert np.array_equal(_bits(a), _bits(b))


@pytest.mark.parametrize("M,N,xdt", [(1031, 17, "bf16"), (9, 4100, "f32")])
def test_split_equals_single_call_and_unaligned_equals_vector(dyt, M, N, xdt):
    log(f"[residual split/unaligned] M={M} N={N} x={xdt}")
    inp, r, dres, d = _setup(M, N, xdt, "f32", 0.9, seed=11)
    h, y = dyt.dyt_forward_residual(d["x"], d["r"], d["alpha"], d["gamma"], d["beta"])
    dh, da, dg, db = dyt.dyt_backward_residual(h, d["dy"], d["dres"], d["alpha"], d["gamma"])
    # split backward
    ws = torch.empty(max(16, dyt.dyt_backward_workspace_size(M, N, xdt, "f32")), dtype=torch.uint8,
                     device="cuda")
    dh2 = torch.empty_like(h)
    da2, dg2, db2 = torch.empty_like(da), torch.empty_like(dg), torch.empty_like(db)
    dyt.dyt_backward_residual_partials(h, d["dy"], d["dres"], d["alpha"], d["gamma"], dh2, ws)
    dyt.dyt_backward_finish(ws, M, N, xdt, da2, dg2, db2)
    # every activation one element off 16-byte alignment: same kernels
    def off(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v
    xu, ru, dyu, dresu = off(d["x"]), off(d["r"]), off(d["dy"]), off(d["dres"])
    hu, yu = off(torch.zeros_like(h)), off(torch.zeros_like(y))
    dyt.dyt_forward_residual(xu, ru, d["alpha"], d["gamma"], d["beta"], h=hu, y=yu)
    dhu = off(torch.zeros_like(dh))
    _, dau, dgu, dbu = dyt.dyt_backward_residual(hu, dyu, dresu, d["alpha"], d["gamma"], dh=dhu)
    torch.cuda.synchronize()
    assert hu.data_ptr() % 16 != 0
    assert np.array_equal(_bits(dh2), _bits(dh))
    for a, b in ((da2, da), (dg2, dg), (db2, db)):
        assert np.array_equal(_bits(a), _bits(b))
    for a, b in ((hu, h), (yu, y), (dhu, dh), (dau, da), (dgu, dg), (dbu, db)):
        assert np.array_equal(_bits(a), _bits(b))
    assert_reports(f"residual {M}x{N}", _reports(inp, r, dres, h, y, dh, da, dg, db))


def test_outputs_stay_inside_their_buffers(dyt):
    """Guard canaries around h, y and dh are untouched."""
    M, N = 777, 45
    inp, r, dres, d = _setup(M, N, "bf16", "f32", 0.5, seed=3)
    canary = -12288.0
    pad = 64

    def guarded():
        buf = torch.full((M * N + 2 * pad,), canary, dtype=torch.bfloat16, device="cuda")
        return buf, buf[pad:pad + M * N].view(M, N)
    hb, h = guarded()
    yb, y = guarded()
    dhb, dh = guarded()
    dyt.dyt_forward_residual(d["x"], d["r"], d["alpha"], d["gamma"], d["beta"], h=h, y=y)
    dyt.dyt_backward_residual(h, d["dy"], d["dres"], d["alpha"], d["gamma"], dh=dh)
    torch.cuda.synchronize()
    for buf in (hb, yb, dhb):
        assert bool((buf[:pad] == canary).all()) and bool((buf[-pad:] == canary).all())


@pytest.mark.parametrize("use_h", [True, False])
def test_residual_module_matches_oracle(dyt, use_h):
    """DyTResidual through autograd: gradients of x and r are dh; with only y
    in the loss (grad_h absent) dh is the plain dx."""
    M, N = 4097, 48
    log(f"[residual module] use_h={use_h}")
    inp, r, dres, d = _setup(M, N, "bf16", "f32", 0.5, seed=17)
    layer = dyt.DyTResidual(N, alpha_init=float(inp.alpha[0]), device="cuda")
    with torch.no_grad():
        layer.weight.copy_(d["gamma"])
        layer.bias.copy_(d["beta"])
    x = d["x"].clone().requires_grad_(True)
    rr = d["r"].clone().requires_grad_(True)
    h, y = layer(x, rr)
    loss = (y.float() * d["dy"].float()).sum()
    if use_h:
        loss = loss + (h.float() * d["dres"].float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    dres_used = dres if use_h else np.zeros_like(dres)
    reps = _reports(inp, r, dres_used, h.detach(), y.detach(), x.grad, layer.alpha.grad,
                    layer.weight.grad, layer.bias.grad)
    assert_reports(f"residual module use_h={use_h}", reps)
    assert np.array_equal(_bits(x.grad), _bits(rr.grad))


@pytest.mark.parametrize("M,N,xdt", [(1031, 300, "bf16"), (64, 4096, "bf16"), (20001, 255, "f32")])
def test_residual_graph_replay_matches_eager(dyt, M, N, xdt):
    """The residual forward and backward captured in one HIP graph replay
    bit-identical to eager calls, replay after replay, with eager work in
    between (the entry points record no memset or allocation)."""
    log(f"[residual graph] M={M} N={N} x={xdt}")
    inp, r, dres, d = _setup(M, N, xdt, "f32", 0.8, seed=5)
    h0, y0 = dyt.dyt_forward_residual(d["x"], d["r"], d["alpha"], d["gamma"], d["beta"])
    ref = (h0, y0) + tuple(dyt.dyt_backward_residual(h0, d["dy"], d["dres"], d["alpha"], d["gamma"]))
    torch.cuda.synchronize()
    h, y, dh = (torch.empty_like(d["x"]) for _ in range(3))
    da, dg, db = torch.empty(1, device="cuda"), torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
    ws = torch.empty(max(16, dyt.dyt_backward_workspace_size(M, N, xdt, "f32")), dtype=torch.uint8,
                     device="cuda")

    def step():
        dyt.dyt_forward_residual(d["x"], d["r"], d["alpha"], d["gamma"], d["beta"], h=h, y=y)
        dyt.dyt_backward_residual(h, d["dy"], d["dres"], d["alpha"], d["gamma"], dh=dh, dalpha=da,
                                  dgamma=dg, dbeta=db, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in (h, y, dh, da, dg, db):
            t.fill_(-7.0)                     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("h", "y", "dh", "dalpha", "dgamma", "dbeta"), (h, y, dh, da, dg, db), ref):
            assert np.array_equal(_bits(got), _bits(want)), f"{name}, replay {rep}"
