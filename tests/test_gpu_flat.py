"""The flat forward: contiguous rows of a whole number of 16-byte vectors
that the slot tiles fill poorly are walked as one run of vectors, with gamma
and beta read from an LDS copy by computed column. Checked against the fp64
oracle element by element, bit for bit against the tiled kernels (a
row-strided launch of the same shape runs the tiles), on problems whose last
vector group is partial, with guard canaries around y, at a base one element
off 16-byte alignment, at the largest width the LDS copy allows, on rows
that are not a whole number of vectors (down to fewer elements than one
vector), and on a problem above 2^31 elements; the residual-fused forward
walks flat in the same way (h exact, y equal to the tiled forward of h)."""
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


CANARY = -12288.0

# (M, N, x dtype, param dtype): every one takes the flat walk (asserted);
# vector groups of 1,024 per workgroup step, the last one partial in most
SHAPES = [
    (1000, 2560, "bf16", "f32"),    # 312.5 groups; row segments 0.62 filled
    (777, 4104, "f32", "f32"),      # 778.5 groups
    (3, 1032, "bf16", "bf16"),      # less than one group; packed tiles of K = 2
    (1, 4100, "f32", "f16"),        # one row: one group and one vector
    (2, 2560, "bf16", "f32"),
    (20000, 1536, "bf16", "f32"),   # packed tiles of K = 2 at 0.75
    (1001, 4104, "bf16", "f32"),
    (129, 1040, "bf16", "f16"),
    (4097, 1032, "f16", "f32"),
    (1234, 4100, "f32", "bf16"),
    (300, 7372, "f32", "f32"),      # 59 KB of LDS
    # float32 rows above 8,192 columns walk flat from 2^26 elements (smaller
    # sizes fill one-slot row segments)
    (5043, 13312, "f32", "f32"),    # above 8,192 columns: 104 KB of LDS
    (3856, 17408, "f32", "bf16"),   # 136 KB of LDS
    (33, 8200, "bf16", "f32"),
    (5001, 32, "bf16", "f32"),      # packed tiles of one full slot (aligned bases only)
    (3001, 64, "f16", "bf16"),
    (999, 256, "bf16", "f32"),
    # rows that are not a whole number of vectors: gamma/beta as 4 shifted
    # copies, the last M*N mod V elements done one by one
    (3001, 1500, "bf16", "f32"),    # 562.7 groups, 4 tail elements
    (777, 17, "bf16", "bf16"),      # 13,209 elements: 1,651 vectors + 1
    (5, 3, "bf16", "f32"),          # N < V: one vector + 7 tail elements
    (1, 7, "f16", "f32"),           # less than one vector: tail only
    (1000, 1501, "f32", "f32"),     # float32 tiles 0.73 filled
    (999, 2039, "f16", "f32"),      # 4 copies of 2,048 words (64 KB of LDS)
    (301, 3575, "bf16", "f32"),     # widest: 4 copies of 3,584 words (112 KB)
    (257, 3071, "bf16", "bf16"),
    (26251, 5113, "f32", "f32"),    # widest float32: 4 copies of 5,120 words (160 KB); 2^27 elements
    (4097, 255, "bf16", "f16"),
]


def _inputs(dyt, M, N, xdt, pdt, seed):
    inp = workloads.custom(M, N, xdt, pdt, alpha=0.7, seed=seed)
    xt, pt = TORCH_DT[xdt], TORCH_DT[pdt]
    x = torch.from_numpy(inp.x).cuda().to(xt)
    a = torch.from_numpy(inp.alpha).cuda().to(pt)
    g = torch.from_numpy(inp.gamma).cuda().to(pt)
    b = torch.from_numpy(inp.beta).cuda().to(pt)
    return inp, x, a, g, b


@pytest.mark.parametrize("M,N,xdt,pdt", SHAPES)
def test_flat_forward_matches_oracle_and_tiles(dyt, M, N, xdt, pdt):
    plan = dyt.dyt_get_forward_plan(M, N, xdt, pdt)
    log(f"[flat] M={M} N={N} x={xdt} p={pdt} plan={plan}")
    assert plan["flat"] == 1 and plan["flat_grid"] >= 1
    inp, x, a, g, b = _inputs(dyt, M, N, xdt, pdt, seed=M * 7 + N)
    xt = TORCH_DT[xdt]

    # contiguous: the flat kernel, y inside a buffer with canaries on both sides
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), CANARY, dtype=xt, device="cuda")
    y = buf[pad:pad + M * N].view(M, N)
    dyt.dyt_forward(x, a, g, b, y=y)
    torch.cuda.synchronize()
    assert bool((buf[:pad] == CANARY).all()) and bool((buf[pad + M * N:] == CANARY).all())
    f = dyt_oracle.forward(inp.x, inp.alpha, inp.gamma, inp.beta)
    assert_reports(f"flat M={M} N={N}", [compare.check_y(to_np(y), f.y, f.scale, xdt)])

    # row-strided launch of the same shape: the tiled kernels, same bits
    xs_buf = torch.full((M, N + 8), CANARY, dtype=xt, device="cuda")
    xs = xs_buf[:, :N]
    xs.copy_(x)
    ys_buf = torch.full((M, N + 16), CANARY, dtype=xt, device="cuda")
    ys = ys_buf[:, :N]
    dyt.dyt_forward(xs, a, g, b, y=ys)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(ys), _bits(y))
    assert bool((ys_buf[:, N:] == CANARY).all())


@pytest.mark.parametrize("M,N,xdt,aligned_only", [
    (1000, 2560, "bf16", 0), (777, 4104, "f32", 0), (4097, 1032, "f16", 0),
    (5001, 32, "bf16", 1), (3001, 64, "f16", 1), (3001, 1500, "bf16", 0), (777, 17, "bf16", 0)])
def test_flat_forward_unaligned_base(dyt, M, N, xdt, aligned_only):
    """x and y one element off 16-byte alignment (both by the same amount:
    the walk starts at their first element on the 128-byte grid, also for
    full one-slot packed tiles): the same bits as aligned."""
    inp, x, a, g, b = _inputs(dyt, M, N, xdt, "f32", seed=N)
    xt = TORCH_DT[xdt]
    plan = dyt.dyt_get_forward_plan(M, N, xdt, "f32")
    log(f"[flat-unaligned] M={M} N={N} x={xdt} plan={plan}")
    assert plan["flat"] == 1 and plan["flat_aligned_only"] == aligned_only
    y = dyt.dyt_forward(x, a, g, b)
    xb = torch.empty(M * N + 1, dtype=xt, device="cuda")
    xu = xb[1:].view(M, N)
    xu.copy_(x)
    yb = torch.full((M * N + 2,), CANARY, dtype=xt, device="cuda")
    yu = yb[1:M * N + 1].view(M, N)
    assert xu.data_ptr() % 16 != 0 and yu.data_ptr() % 16 != 0
    dyt.dyt_forward(xu, a, g, b, y=yu)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(yu), _bits(y))
    assert float(yb[0]) == CANARY and float(yb[-1]) == CANARY
    f = dyt_oracle.forward(inp.x, inp.alpha, inp.gamma, inp.beta)
    assert_reports(f"flat unaligned M={M} N={N}", [compare.check_y(to_np(yu), f.y, f.scale, xdt)])


@pytest.mark.parametrize("M,N,xdt,xo,yo", [
    (1000, 2560, "bf16", 1, 3), (3001, 1500, "bf16", 2, 0), (777, 4104, "f32", 0, 1), (5, 3, "bf16", 3, 3),
    (1, 5, "bf16", 5, 5), (1000, 2560, "bf16", 1, 9), (777, 4104, "f32", 1, 5), (999, 1500, "bf16", 7, 7),
    (5001, 32, "bf16", 1, 3), (5001, 32, "bf16", 3, 3),   # one-slot packed: tiles, then the shifted walk
    # rows over 8,192 columns (gamma/beta in 104-160 KB of LDS; no shifted copies fit, so
    # these walk unaligned from element 0)
    (5043, 13312, "f32", 1, 1), (5043, 13312, "f32", 1, 2), (33, 8200, "bf16", 1, 3),
    (33, 8200, "bf16", 5, 5), (7, 20480, "f32", 3, 0)])
def test_flat_forward_other_misalignments(dyt, M, N, xdt, xo, yo):
    """x and y off the 16-byte grid by xo and yo elements (equal offsets
    within a 128-byte line: the walk starts on the line grid; equal only
    within 16 bytes: on the 16-byte grid; else it runs unaligned): the same
    bits as the aligned call, canaries around y untouched."""
    inp, x, a, g, b = _inputs(dyt, M, N, xdt, "f32", seed=N + xo)
    xt = TORCH_DT[xdt]
    log(f"[flat-misaligned] M={M} N={N} x={xdt} xo={xo} yo={yo}")
    y = dyt.dyt_forward(x, a, g, b)
    xb = torch.empty(M * N + 8, dtype=xt, device="cuda")
    xu = xb[xo:xo + M * N].view(M, N)
    xu.copy_(x)
    yb = torch.full((M * N + 16,), CANARY, dtype=xt, device="cuda")
    yu = yb[yo:yo + M * N].view(M, N)
    dyt.dyt_forward(xu, a, g, b, y=yu)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(yu), _bits(y))
    assert bool((yb[:yo] == CANARY).all()) and bool((yb[yo + M * N:] == CANARY).all())


def test_flat_forward_repeat_is_bitwise_stable(dyt):
    M, N = 1001, 4104
    _, x, a, g, b = _inputs(dyt, M, N, "bf16", "f32", seed=5)
    y1 = dyt.dyt_forward(x, a, g, b)
    y2 = dyt.dyt_forward(x, a, g, b)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y1), _bits(y2))


def test_flat_forward_above_2_31_elements(dyt):
    """838,865 x 2,560 bfloat16 (2.15e9 elements, 64-bit vector offsets):
    y against the oracle on sampled elements around element 2^31 and at the
    end, and equal to the tiled (row-strided) launch there."""
    M, N = 838865, 2560
    total = M * N
    assert total > 2 ** 31
    free, _ = torch.cuda.mem_get_info()
    if free < 24 * 2 ** 30:
        pytest.skip("needs ~24 GB of free device memory")
    plan = dyt.dyt_get_forward_plan(M, N, "bf16", "f32")
    log(f"[flat large] M={M} N={N} plan={plan}")
    assert plan["flat"] == 1
    gen = torch.Generator(device="cuda").manual_seed(17)
    x = torch.randn(M, N, generator=gen, device="cuda", dtype=torch.bfloat16)
    gamma = torch.rand(N, generator=gen, device="cuda") + 0.5
    beta = torch.randn(N, generator=gen, device="cuda") * 0.1
    alpha = torch.full((1,), 0.8, device="cuda")
    y = dyt.dyt_forward(x, alpha, gamma, beta)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    idx = np.unique(np.concatenate([rng.integers(0, total, 1 << 18),
                                    np.arange(2 ** 31 - 4096, 2 ** 31 + 4096),
                                    np.arange(total - 4096, total)]))
    assert idx[0] >= 0 and idx[-1] < total
    it = torch.from_numpy(idx).cuda()
    xs = to_np(x.view(-1)[it])
    cols = idx % N
    ys, ss = dyt_oracle.forward_at(xs, cols, [0.8], to_np(gamma), to_np(beta))
    got = y.view(-1)[it]
    assert_reports("flat large y", [compare.check_y(to_np(got), ys, ss, "bf16")])
    # the tiled kernels on the rows around element 2^31 and the last rows
    for r0 in ((2 ** 31) // N - 2, M - 3):
        xs_buf = torch.empty((3, N + 8), dtype=torch.bfloat16, device="cuda")
        xv = xs_buf[:, :N]
        xv.copy_(x[r0:r0 + 3])
        ys_buf = torch.empty((3, N + 8), dtype=torch.bfloat16, device="cuda")
        yv = ys_buf[:, :N]
        dyt.dyt_forward(xv, alpha, gamma, beta, y=yv)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(yv), _bits(y[r0:r0 + 3]))
    del x, y
    torch.cuda.empty_cache()


RES_SHAPES = [  # residual-fused forward: every one walks flat (asserted)
    (1000, 2560, "bf16", "f32"),
    (4099, 3072, "bf16", "bf16"),   # tiles 0.75 filled: the plain forward keeps them, this one not
    (777, 4104, "f32", "f32"),
    (129, 1040, "bf16", "f16"),
    (3, 1032, "f16", "f32"),
    (300, 7372, "f32", "f32"),
    # rows that are not a whole number of vectors
    (3001, 1500, "bf16", "f32"),
    (777, 17, "bf16", "bf16"),
    (5, 3, "f16", "f32"),           # one vector + 7 tail elements
    (1000, 1501, "f32", "f32"),
]


@pytest.mark.parametrize("M,N,xdt,pdt", RES_SHAPES)
def test_flat_residual_forward(dyt, M, N, xdt, pdt):
    """h = x + r exactly the oracle's rounded sum, y within tolerance of the
    oracle on h and bit for bit the tiled forward of h (row-strided launch);
    canaries around h and y untouched."""
    plan = dyt.dyt_get_forward_residual_plan(M, N, xdt, pdt)
    log(f"[flat residual] M={M} N={N} x={xdt} p={pdt} plan={plan}")
    assert plan["flat"] == 1
    inp = workloads.custom(M, N, xdt, pdt, alpha=0.6, seed=N + 3 * M)
    r, _ = workloads.residual_pair(M, N, xdt, N)
    xt, pt = TORCH_DT[xdt], TORCH_DT[pdt]
    x = torch.from_numpy(inp.x).cuda().to(xt)
    rt = torch.from_numpy(np.ascontiguousarray(r)).cuda().to(xt)
    a = torch.from_numpy(inp.alpha).cuda().to(pt)
    g = torch.from_numpy(inp.gamma).cuda().to(pt)
    b = torch.from_numpy(inp.beta).cuda().to(pt)
    pad = 2048
    hb = torch.full((M * N + 2 * pad,), CANARY, dtype=xt, device="cuda")
    yb = torch.full((M * N + 2 * pad,), CANARY, dtype=xt, device="cuda")
    h = hb[pad:pad + M * N].view(M, N)
    y = yb[pad:pad + M * N].view(M, N)
    dyt.dyt_forward_residual(x, rt, a, g, b, h=h, y=y)
    torch.cuda.synchronize()
    for buf in (hb, yb):
        assert bool((buf[:pad] == CANARY).all()) and bool((buf[pad + M * N:] == CANARY).all())
    h_ref, f = dyt_oracle.forward_residual(inp.x, r, inp.alpha, inp.gamma, inp.beta, xdt)
    assert_reports(f"flat residual M={M} N={N}",
                   [compare.check_exact(to_np(h), h_ref, "h"),
                    compare.check_y(to_np(y), f.y, f.scale, xdt)])
    hs_buf = torch.empty((M, N + 8), dtype=xt, device="cuda")
    hs = hs_buf[:, :N]
    hs.copy_(h)
    ys_buf = torch.empty((M, N + 8), dtype=xt, device="cuda")
    ys = ys_buf[:, :N]
    dyt.dyt_forward(hs, a, g, b, y=ys)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(ys), _bits(y))


@pytest.mark.parametrize("M,N,xdt", [(1000, 2560, "bf16"), (777, 4104, "f32")])
def test_flat_forward_ieee_special_values(dyt, M, N, xdt):
    """alpha = +inf on a flat shape: real elements with x = 0 give NaN
    (tanh(inf * 0)), float32 subnormal x gives +-gamma + beta (no flush),
    every other element +-gamma + beta; matches the oracle element by element
    and the tiled kernels bit for bit."""
    inp = workloads.custom(M, N, xdt, "f32", alpha=float("inf"), seed=N + 1)
    x = inp.x.copy()
    rng = np.random.default_rng(5)
    zi = rng.integers(0, M * N, 64)
    x.reshape(-1)[zi] = 0.0
    if xdt == "f32":
        si = rng.integers(0, M * N, 64)
        si = si[~np.isin(si, zi)]
        x.reshape(-1)[si] = np.float32(1e-41) * np.where(rng.random(si.size) < 0.5, -1, 1).astype(np.float32)
    assert dyt.dyt_get_forward_plan(M, N, xdt, "f32")["flat"] == 1
    xt = TORCH_DT[xdt]
    xg = torch.from_numpy(x).cuda().to(xt)
    a = torch.full((1,), float("inf"), device="cuda")
    g = torch.from_numpy(inp.gamma).cuda()
    b = torch.from_numpy(inp.beta).cuda()
    y = dyt.dyt_forward(xg, a, g, b)
    xs_buf = torch.empty((M, N + 8), dtype=xt, device="cuda")
    xs = xs_buf[:, :N]
    xs.copy_(xg)
    ys_buf = torch.empty((M, N + 8), dtype=xt, device="cuda")
    ys = ys_buf[:, :N]
    dyt.dyt_forward(xs, a, g, b, y=ys)
    torch.cuda.synchronize()
    f = dyt_oracle.forward(x, [np.inf], inp.gamma, inp.beta)
    assert_reports(f"flat alpha=inf M={M} N={N}", [compare.check_y(to_np(y), f.y, f.scale, xdt)])
    yn = to_np(y)
    assert np.isnan(yn.reshape(-1)[zi]).all() and np.isnan(yn).sum() == np.unique(zi).size
    assert np.array_equal(_bits(ys), _bits(y))


@pytest.mark.parametrize("M,N,packed", [
    (20000, 4096, 0),    # four full one-slot row segments per row
    (700000, 100, 1),    # packed rows
    (270000, 255, 1),    # packed rows that are not a whole number of vectors
])
def test_large_float32_rows_walk_flat(dyt, M, N, packed):
    """Float32 rows beyond 2^26 elements walk flat however full their tiles,
    while the same rows at 2^26 elements keep their tiles; y equals the
    tiled (row-strided) launch bit for bit and the oracle on sampled
    elements."""
    plan = dyt.dyt_get_forward_plan(M, N, "f32", "f32")
    log(f"[flat large f32] M={M} N={N} plan={plan}")
    assert M * N > 1 << 26
    assert plan["flat"] == 1 and plan["packed"] == packed
    assert dyt.dyt_get_forward_plan((1 << 26) // N, N, "f32", "f32")["flat"] == 0
    inp, x, a, g, b = _inputs(dyt, M, N, "f32", "f32", seed=N)
    y = dyt.dyt_forward(x, a, g, b)
    xs_buf = torch.empty((M, N + 8), device="cuda")
    xs = xs_buf[:, :N]
    xs.copy_(x)
    ys_buf = torch.full((M, N + 8), CANARY, device="cuda")
    ys = ys_buf[:, :N]
    dyt.dyt_forward(xs, a, g, b, y=ys)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(ys), _bits(y))
    assert bool((ys_buf[:, N:] == CANARY).all())
    rng = np.random.default_rng(3)
    total = M * N
    idx = np.unique(np.concatenate([rng.integers(0, total, size=1 << 18), np.arange(4096),
                                    np.arange(total - 4096, total)]))
    rows, cols = np.divmod(idx, N)
    ref, scale = dyt_oracle.forward_at(inp.x[rows, cols], cols, inp.alpha, inp.gamma, inp.beta)
    y_s = to_np(y.reshape(-1)[torch.from_numpy(idx).cuda()])
    assert_reports(f"flat large f32 M={M} N={N}", [compare.check_y(y_s, ref, scale, "f32", "y[sampled]")])
