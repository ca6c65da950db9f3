"""Properties of the HIP path that hold exactly (bitwise), independent of the
oracle's tolerances: run-to-run determinism, exact power-of-two scaling,
poisoned tails and guard canaries (no NaN leakage from padding, no writes
outside the outputs), closed forms (alpha = 0, alpha = +inf with integer
data), odd symmetry in x and in alpha, subnormal inputs, and tensors at
bases aligned only to the element size giving the same bits as 16-byte
aligned ones."""
import os

import numpy as np
import pytest
import torch

import workloads
from gpu_util import TORCH_DT, assert_reports, full_reports, log, run_both, to_np, upload

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


def test_in_tree_library_is_the_one_loaded(dyt):
    maps = open("/proc/self/maps").read()
    assert os.path.realpath(dyt.LIB_FILE) in maps


CASES = [("c5_4194304x32_bf16_outliers", 20001), ("c4_32768x4096_bf16", 64),
         ("c3_100003x17_f32_inf", 5003), ("c2_65537x16_bf16", 65537), ("c1_1024x64_f32", 1024)]


@pytest.mark.parametrize("name,M", CASES)
def test_bitwise_deterministic(dyt, name, M):
    log(f"[determinism] {name} M={M}")
    d = upload(workloads.generate(name, M=M))
    a = run_both(dyt, d)
    b = run_both(dyt, d)
    for u, v in zip(a, b):
        assert np.array_equal(_bits(u), _bits(v))


@pytest.mark.parametrize("name,M", [("c4_32768x4096_bf16", 33), ("c2_65537x16_bf16", 4097),
                                   ("c1_1024x64_f32", 1024)])
def test_dy_times_two_scales_every_output_exactly(dyt, name, M):
    d = upload(workloads.generate(name, M=M))
    _, dx1, da1, dg1, db1 = run_both(dyt, d)
    d2 = dict(d, dy=d["dy"] * 2)
    _, dx2, da2, dg2, db2 = run_both(dyt, d2)
    for u, v in ((dx1, dx2), (da1, da2), (dg1, dg2), (db1, db2)):
        assert np.array_equal(_bits(u * 2), _bits(v))


def _embedded(t: torch.Tensor, pad_before: int, pad_after: int, fill: float):
    """Copy t into a larger flat buffer (fill around it); return (view, buffer)."""
    n = t.numel()
    buf = torch.full((pad_before + n + pad_after,), fill, dtype=t.dtype, device=t.device)
    view = buf[pad_before:pad_before + n].view(t.shape)
    view.copy_(t)
    return view, buf


@pytest.mark.parametrize("name,M", [("c3_100003x17_f32_inf", 1003), ("c3_100003x255_f32_inf", 333),
                                    ("c5_4194304x32_bf16_outliers", 999), ("c2_65537x16_bf16", 3001)])
def test_poisoned_tail_and_canaries(dyt, name, M):
    """Inputs followed by NaN/inf in the same allocation give the same bits as
    clean inputs, and guard regions around every output stay untouched."""
    log(f"[poison] {name} M={M}")
    d = upload(workloads.generate(name, M=M))
    ref = run_both(dyt, d)
    sx = d["x"].element_size()
    pad = 64 // sx                                # 64 bytes: keeps 16-byte alignment
    for fill in (float("nan"), float("inf"), 0.0):
        x, _ = _embedded(d["x"], pad, pad, fill)
        dy, _ = _embedded(d["dy"], pad, pad, fill)
        canary = -12288.0                      # exact in bfloat16 and float32
        y, ybuf = _embedded(torch.empty_like(d["x"]), pad, pad, canary)
        dx, dxbuf = _embedded(torch.empty_like(d["x"]), pad, pad, canary)
        pdt = d["alpha"].dtype
        N = d["x"].shape[1]
        dg, dgbuf = _embedded(torch.empty(N, dtype=pdt, device="cuda"), 16, 16, canary)
        db, dbbuf = _embedded(torch.empty(N, dtype=pdt, device="cuda"), 16, 16, canary)
        da, dabuf = _embedded(torch.empty(1, dtype=pdt, device="cuda"), 16, 16, canary)
        need = dyt.dyt_backward_workspace_size(*d["x"].shape, d["x"].dtype, pdt)
        ws, wsbuf = _embedded(torch.empty(need // 4, dtype=torch.float32, device="cuda"), 64, 64, canary)
        dyt.dyt_forward(x, d["alpha"], d["gamma"], d["beta"], y=y)
        dyt.dyt_backward(x, dy, d["alpha"], d["gamma"], dx=dx, dalpha=da, dgamma=dg, dbeta=db,
                         workspace=ws)
        torch.cuda.synchronize()
        for got, want in zip((y, dx, da, dg, db), ref):
            assert np.array_equal(_bits(got), _bits(want)), f"fill={fill}"
        for buf, p in ((ybuf, pad), (dxbuf, pad), (dgbuf, 16), (dbbuf, 16), (dabuf, 16), (wsbuf, 64)):
            assert bool((buf[:p] == canary).all()) and bool((buf[-p:] == canary).all()), "canary hit"


def test_alpha_zero_closed_form(dyt):
    """alpha = 0: y = beta exactly, dx = 0, dgamma = 0; integer data makes
    dbeta and dalpha exact integers."""
    rng = np.random.default_rng(11)
    M, N = 5003, 100
    x = rng.integers(-2, 3, size=(M, N)).astype(np.float32)
    dy = rng.integers(-3, 4, size=(M, N)).astype(np.float32)
    g = rng.integers(1, 3, size=N).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    for xdt in ("f32", "bf16"):
        inp = workloads.from_arrays(x, dy, [0.0], g, b, xdt, "f32")
        y, dx, da, dg, db = run_both(dyt, upload(inp))
        assert np.array_equal(to_np(y), np.broadcast_to(b.astype(np.float64), (M, N)) if xdt == "f32"
                              else np.broadcast_to(to_np(torch.from_numpy(b).to(torch.bfloat16)), (M, N)))
        assert not to_np(dx).any() and not to_np(dg).any()
        want_db = dy.astype(np.int64).sum(axis=0)
        want_da = int((dy.astype(np.int64) * g.astype(np.int64) * x.astype(np.int64)).sum())
        assert np.array_equal(to_np(db), want_db.astype(np.float64))
        assert to_np(da)[0] == want_da


@pytest.mark.parametrize("N", [17, 100, 255])
def test_alpha_inf_integer_sums_exact(dyt, N):
    """alpha = +inf, nonzero x, integer dy (M = 100,003): dgamma = sum dy*sign(x)
    and dbeta = sum dy exactly, dalpha = 0, dx NaN everywhere (no NaN leaks
    into the sums from the ragged last tile)."""
    rng = np.random.default_rng(N)
    M = 100003
    x = (rng.standard_normal((M, N)) * 2).astype(np.float32)
    x[x == 0] = 1.0
    dy = rng.integers(-3, 4, size=(M, N)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, N).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    inp = workloads.from_arrays(x, dy, [np.inf], g, b, "f32", "f32")
    y, dx, da, dg, db = run_both(dyt, upload(inp))
    sgn = np.where(x > 0, 1, -1).astype(np.int64)
    assert np.array_equal(to_np(dg), (dy.astype(np.int64) * sgn).sum(axis=0).astype(np.float64))
    assert np.array_equal(to_np(db), dy.astype(np.int64).sum(axis=0).astype(np.float64))
    assert to_np(da)[0] == 0.0
    assert np.isnan(to_np(dx)).all()
    yy = to_np(y)
    assert np.array_equal(yy, (np.where(x > 0, g, -g) + b).astype(np.float32).astype(np.float64))


def test_alpha_inf_real_zero_gives_nan_only_where_ieee_says(dyt):
    """x = 0 in a real row with alpha = +inf: y, that column's dgamma and
    dalpha are NaN (IEEE: inf * 0); every other column stays finite."""
    inp = workloads.generate("c3_100003x17_f32_inf", M=2000)
    inp.x[1234, 5] = 0.0
    inp.x[7, 11] = -0.0
    y, dx, da, dg, db = run_both(dyt, upload(inp))
    yy = to_np(y)
    assert np.isnan(yy[1234, 5]) and np.isnan(yy[7, 11])
    assert np.isfinite(np.delete(yy.reshape(-1), [1234 * 17 + 5, 7 * 17 + 11])).all()
    dgg = to_np(dg)
    assert np.isnan(dgg[[5, 11]]).all() and np.isfinite(np.delete(dgg, [5, 11])).all()
    assert np.isfinite(to_np(db)).all()
    assert np.isnan(to_np(da)[0])
    assert_reports("alpha-inf zeros", full_reports(inp, y, dx, da, dg, db))


def test_subnormal_x_with_infinite_alpha(dyt):
    """float32 subnormal x with alpha = +inf is not flushed: y = +-gamma + beta."""
    M, N = 64, 16
    x = np.full((M, N), 2.0 ** -140, dtype=np.float32)
    x[::2] *= -1
    dy = np.ones((M, N), dtype=np.float32)
    g = np.linspace(0.5, 1.5, N).astype(np.float32)
    b = np.linspace(-0.1, 0.1, N).astype(np.float32)
    inp = workloads.from_arrays(x, dy, [np.inf], g, b, "f32", "f32")
    y, dx, da, dg, db = run_both(dyt, upload(inp))
    want = np.where(x > 0, g, -g) + b
    assert np.array_equal(to_np(y), want.astype(np.float32).astype(np.float64))
    assert to_np(da)[0] == 0.0


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_odd_symmetry_bitwise(dyt, xdt):
    inp = workloads.custom(999, 64, xdt, "f32", alpha=0.9, x_sigma=3.0, seed=5)
    inp.beta[:] = 0
    d = upload(inp)
    y1 = dyt.dyt_forward(d["x"], d["alpha"], d["gamma"], d["beta"])
    y2 = dyt.dyt_forward(-d["x"], d["alpha"], d["gamma"], d["beta"])
    torch.cuda.synchronize()
    assert np.array_equal(_bits(-y1), _bits(y2))


@pytest.mark.parametrize("M,N,xdt,pdt", [
    (100003, 255, "f32", "f32"),    # packed tiles of two slots
    (300, 4096, "bf16", "f32"),     # row segments
    (1000, 2560, "bf16", "f32"),    # the flat forward
    (1031, 300, "f16", "f16"),
    (41, 4100, "f32", "bf16"),      # rows that are not a whole number of vectors
])
def test_negated_alpha_bitwise(dyt, M, N, xdt, pdt):
    """alpha -> -alpha: tanh is odd and sech^2 even, and rounding to nearest
    is symmetric, so y(x, -alpha) equals y(-x, alpha), dx and dgamma change
    sign, and dbeta and dalpha stay the same, all bit for bit."""
    log(f"[negated alpha] M={M} N={N} x={xdt} p={pdt}")
    inp = workloads.custom(M, N, xdt, pdt, alpha=0.7, x_sigma=2.0, seed=N)
    d = upload(inp)
    na = -d["alpha"]
    y1 = dyt.dyt_forward(d["x"], na, d["gamma"], d["beta"])
    y2 = dyt.dyt_forward(-d["x"], d["alpha"], d["gamma"], d["beta"])
    g1 = dyt.dyt_backward(d["x"], d["dy"], d["alpha"], d["gamma"])
    g2 = dyt.dyt_backward(d["x"], d["dy"], na, d["gamma"])
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y1), _bits(y2))
    dx1, da1, dg1, db1 = g1
    dx2, da2, dg2, db2 = g2
    assert np.array_equal(_bits(dx2), _bits(-dx1))
    assert np.array_equal(_bits(dg2), _bits(-dg1))
    assert np.array_equal(_bits(db2), _bits(db1))
    assert np.array_equal(_bits(da2), _bits(da1))


@pytest.mark.parametrize("name,M", [("c2_65537x16_bf16", 4097), ("c1_1024x64_f32", 1024),
                                    ("c4_32768x4096_bf16", 17), ("c3_100003x100_f32_inf", 999)])
def test_unaligned_bases_equal_aligned(dyt, name, M):
    """Bases aligned only to the element size run the same 16-byte kernels
    and tiles: every output, gradients included, is bitwise equal to the
    aligned call's (and matches the oracle)."""
    inp = workloads.generate(name, M=M)
    d = upload(inp)
    ref = run_both(dyt, d)
    x, _ = _embedded(d["x"], 1, 0, 0.0)
    dy, _ = _embedded(d["dy"], 1, 0, 0.0)
    y, _ = _embedded(torch.empty_like(d["x"]), 1, 0, 0.0)
    dx, _ = _embedded(torch.empty_like(d["x"]), 1, 0, 0.0)
    assert x.data_ptr() % 16 != 0
    dyt.dyt_forward(x, d["alpha"], d["gamma"], d["beta"], y=y)
    _, da, dg, db = dyt.dyt_backward(x, dy, d["alpha"], d["gamma"], dx=dx)
    torch.cuda.synchronize()
    for u, v in zip((y, dx, da, dg, db), ref):
        assert np.array_equal(_bits(u), _bits(v))
    assert_reports(f"{name} unaligned", full_reports(inp, y, dx, da, dg, db))


def test_empty_problems(dyt):
    for xdt in ("f32", "bf16"):
        t = TORCH_DT[xdt]
        x = torch.empty(0, 8, dtype=t, device="cuda")
        a = torch.ones(1, device="cuda")
        g = torch.ones(8, device="cuda")
        y = dyt.dyt_forward(x, a, g, g)
        assert y.shape == (0, 8)
        dg = torch.full((8,), 7.0, device="cuda")
        db = torch.full((8,), 7.0, device="cuda")
        da = torch.full((1,), 7.0, device="cuda")
        dyt.dyt_backward(x, x, a, g, dgamma=dg, dbeta=db, dalpha=da)
        torch.cuda.synchronize()
        assert not dg.any() and not db.any() and not da.any()
        x = torch.empty(5, 0, dtype=t, device="cuda")
        da = torch.full((1,), 7.0, device="cuda")
        dyt.dyt_backward(x, x, a, torch.ones(0, device="cuda"), dalpha=da)
        torch.cuda.synchronize()
        assert not da.any()


def test_large_u_float32_keeps_sech2(dyt):
    """|alpha x| up to 60 in float32: sech^2 is taken without cancellation, so
    dx stays within 1e-6 relative where 1 - tanh^2 would give 0."""
    M, N = 256, 64
    x = np.linspace(-60, 60, M * N, dtype=np.float32).reshape(M, N)
    inp = workloads.from_arrays(x, np.ones((M, N), np.float32), [1.0], np.ones(N, np.float32),
                                np.zeros(N, np.float32), "f32", "f32")
    outs = run_both(dyt, upload(inp))
    assert_reports("large-u f32", full_reports(inp, *outs))


@pytest.mark.parametrize("name,M", [("c5_4194304x32_bf16_outliers", 20001), ("c4_32768x4096_bf16", 40),
                                    ("c3_100003x17_f32_inf", 3001)])
def test_split_backward_matches_single_call(dyt, name, M):
    """dyt_backward_partials + dyt_backward_finish == dyt_backward, bitwise."""
    d = upload(workloads.generate(name, M=M))
    _, dx0, da0, dg0, db0 = run_both(dyt, d)
    x = d["x"]
    Mx, N = x.shape
    pdt = d["alpha"].dtype
    dx = torch.empty_like(x)
    ws = torch.empty(dyt.dyt_backward_workspace_size(Mx, N, x.dtype, pdt), dtype=torch.uint8, device="cuda")
    da = torch.empty(1, dtype=pdt, device="cuda")
    dg = torch.empty(N, dtype=pdt, device="cuda")
    db = torch.empty(N, dtype=pdt, device="cuda")
    dyt.dyt_backward_partials(x, d["dy"], d["alpha"], d["gamma"], dx, ws)
    dyt.dyt_backward_finish(ws, Mx, N, x.dtype, da, dg, db)
    torch.cuda.synchronize()
    for u, v in ((dx, dx0), (da, da0), (dg, dg0), (db, db0)):
        assert np.array_equal(_bits(u), _bits(v))


@pytest.mark.parametrize("name,M", [("c2_65537x16_bf16", 65537), ("c4_32768x4096_bf16", 40),
                                    ("c3_100003x17_f32_inf", 2001)])
def test_hip_graph_replay_matches_eager(dyt, name, M):
    """A forward + backward step captured in a HIP graph replays bit-identical
    to eager execution, replay after replay, with eager work in between (the
    kernels record no memset or allocation into the graph)."""
    log(f"[graph] {name} M={M}")
    d = upload(workloads.generate(name, M=M))
    ref = run_both(dyt, d)
    x = d["x"]
    Mx, N = x.shape
    pdt = d["alpha"].dtype
    y, dx = torch.empty_like(x), torch.empty_like(x)
    da = torch.empty(1, dtype=pdt, device="cuda")
    dg = torch.empty(N, dtype=pdt, device="cuda")
    db = torch.empty(N, dtype=pdt, device="cuda")
    ws = torch.empty(dyt.dyt_backward_workspace_size(Mx, N, x.dtype, pdt), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dyt.dyt_forward(x, d["alpha"], d["gamma"], d["beta"], y=y)
        dyt.dyt_backward(x, d["dy"], d["alpha"], d["gamma"], dx=dx, dalpha=da, dgamma=dg, dbeta=db, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dyt.dyt_forward(x, d["alpha"], d["gamma"], d["beta"], y=y)
        dyt.dyt_backward(x, d["dy"], d["alpha"], d["gamma"], dx=dx, dalpha=da, dgamma=dg, dbeta=db, workspace=ws)
    for rep in range(4):
        for t in (y, dx, da, dg, db):
            t.fill_(-7.0)                     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((y, dx, da, dg, db), ref):
            assert np.array_equal(_bits(got), _bits(want)), f"replay {rep}"
