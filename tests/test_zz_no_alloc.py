"""The allocation-free backward entry point (static device scratch) against
dyt_backward with a caller workspace: same kernels, so equal bit for bit, on
two calls in a row, the second with a smaller problem, through the C ABI."""
import pytest
import torch

from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dyt():
    import __graft_entry__ as ge
    ge._ensure_built()
    import bwd_dyt_forward_amd as m
    return m


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _inputs(M, N, xdt, pdt, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = (2 * torch.randn(M, N, device="cuda", generator=g)).to(xdt)
    dy = torch.randn(M, N, device="cuda", generator=g).to(xdt)
    a = torch.tensor([0.7], device="cuda").to(pdt)
    gm = (1 + 0.1 * torch.randn(N, device="cuda", generator=g)).to(pdt)
    return x, dy, a, gm


def _noalloc_raw(dyt, x, dy, a, gm, dx, da, dg, db):
    """Straight through the C ABI (ctypes), no Python-side checks."""
    L = dyt.lib
    M, N = x.shape
    s = torch.cuda.current_stream().cuda_stream
    return L.dyt_backward_noalloc(x.data_ptr(), dy.data_ptr(), a.data_ptr(), gm.data_ptr(), dx.data_ptr(),
                                  da.data_ptr(), dg.data_ptr(), db.data_ptr(), M, N,
                                  dyt._lib._code(x.dtype), dyt._lib._code(a.dtype), s)


# (M, N, x dtype, param dtype) pairs: the first call, then a smaller one
CASES = [
    ((32768, 4096, torch.bfloat16, torch.float32), (1000, 4096, torch.bfloat16, torch.float32)),
    ((4194304, 32, torch.bfloat16, torch.float32), (65537, 16, torch.bfloat16, torch.float32)),
    ((100003, 255, torch.float32, torch.float32), (1024, 64, torch.float32, torch.float32)),
    ((1000, 18430, torch.bfloat16, torch.float32), (7, 4100, torch.float16, torch.bfloat16)),
]


@pytest.mark.parametrize("first,second", CASES, ids=lambda c: f"{c[0]}x{c[1]}")
def test_noalloc_equals_workspace_backward_twice(dyt, first, second):
    for k, (M, N, xdt, pdt) in enumerate((first, second)):
        log(f"[noalloc] call {k + 1}: M={M} N={N} x={xdt} p={pdt}")
        x, dy, a, gm = _inputs(M, N, xdt, pdt, seed=M + N + k)
        ref = dyt.dyt_backward(x, dy, a, gm)
        outs = (torch.full_like(x, float("nan")), torch.full((1,), float("nan"), dtype=pdt, device="cuda"),
                torch.full((N,), float("nan"), dtype=pdt, device="cuda"),
                torch.full((N,), float("nan"), dtype=pdt, device="cuda"))
        assert _noalloc_raw(dyt, x, dy, a, gm, *outs) == 0
        torch.cuda.synchronize()
        for name, r, o in zip(("dx", "dalpha", "dgamma", "dbeta"), ref, outs):
            assert torch.equal(_bits(r), _bits(o)), f"{name} differs (call {k + 1}, M={M}, N={N})"
        del x, dy, ref, outs
    torch.cuda.empty_cache()


def test_noalloc_binding_and_empty_problems(dyt):
    x, dy, a, gm = _inputs(513, 17, torch.float32, torch.float32, seed=3)
    dx, da, dg, db = torch.empty_like(x), torch.empty(1, device="cuda"), torch.empty(17, device="cuda"), \
        torch.empty(17, device="cuda")
    dyt.dyt_backward_noalloc(x, dy, a, gm, dx, da, dg, db)
    ref = dyt.dyt_backward(x, dy, a, gm)
    torch.cuda.synchronize()
    for r, o in zip(ref, (dx, da, dg, db)):
        assert torch.equal(_bits(r), _bits(o))
    # M = 0: the gradients are empty sums
    e = torch.empty(0, 17, device="cuda")
    da.fill_(5.0); dg.fill_(5.0); db.fill_(5.0)
    dyt.dyt_backward_noalloc(e, e, a, gm, e, da, dg, db)
    torch.cuda.synchronize()
    assert float(da[0]) == 0.0 and bool((dg == 0).all()) and bool((db == 0).all())


def test_noalloc_rejects_problems_beyond_the_scratch(dyt):
    # one row of 2^22 float32 columns: 2,048 column blocks of partial rows, 32 MiB
    M, N = 1, 1 << 22
    assert dyt.dyt_backward_workspace_size(M, N, "f32", "f32") > dyt._lib.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(M, N, device="cuda")
    p = torch.zeros(N, device="cuda")
    with pytest.raises(dyt.DytError) as e:
        dyt.dyt_backward_noalloc(x, x, p[:1], p, torch.empty_like(x), p[:1].clone(), p.clone(), p.clone())
    assert e.value.status == 3   # DYT_ERR_WORKSPACE_TOO_SMALL


def test_noalloc_over_a_sequence_of_problems(dyt):
    """Sixteen seeded problems in a row (widths log-uniform in 1 .. 20,000,
    up to 2^22 elements, every dtype pair), sizes going up and down, so the
    shared scratch holds an earlier, larger or smaller problem's partial rows
    when each call starts: each equals dyt_backward bit for bit."""
    import math
    import numpy as np
    rng = np.random.default_rng(20251203)
    dts = [torch.float32, torch.bfloat16, torch.float16]
    for k in range(16):
        N = int(round(math.exp(rng.uniform(0.0, math.log(20000.0)))))
        M = max(1, int(rng.integers(1 << 8, 1 << 22)) // N)
        xdt, pdt = dts[int(rng.integers(0, 3))], dts[int(rng.integers(0, 3))]
        log(f"[noalloc sequence] call {k + 1}: M={M} N={N} x={xdt} p={pdt}")
        x, dy, a, gm = _inputs(M, N, xdt, pdt, seed=500 + k)
        ref = dyt.dyt_backward(x, dy, a, gm)
        outs = (torch.full_like(x, float("nan")), torch.full((1,), float("nan"), dtype=pdt, device="cuda"),
                torch.full((N,), float("nan"), dtype=pdt, device="cuda"),
                torch.full((N,), float("nan"), dtype=pdt, device="cuda"))
        assert _noalloc_raw(dyt, x, dy, a, gm, *outs) == 0
        torch.cuda.synchronize()
        for name, r, o in zip(("dx", "dalpha", "dgamma", "dbeta"), ref, outs):
            assert torch.equal(_bits(r), _bits(o)), f"{name} differs (call {k + 1}, M={M}, N={N})"


@pytest.mark.parametrize("M,N,xdt", [(100003, 255, torch.float32), (1000, 4096, torch.bfloat16)])
def test_noalloc_graph_replay_matches_eager(dyt, M, N, xdt):
    """Callers that cannot allocate include code under HIP graph capture: the
    allocation-free backward captured in a graph replays bit-identical to
    dyt_backward, replay after replay, with eager work in between."""
    log(f"[noalloc graph] M={M} N={N} x={xdt}")
    x, dy, a, gm = _inputs(M, N, xdt, torch.float32, seed=77)
    ref = dyt.dyt_backward(x, dy, a, gm)
    torch.cuda.synchronize()
    outs = (torch.empty_like(x), torch.empty(1, device="cuda"), torch.empty(N, device="cuda"),
            torch.empty(N, device="cuda"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        assert _noalloc_raw(dyt, x, dy, a, gm, *outs) == 0
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert _noalloc_raw(dyt, x, dy, a, gm, *outs) == 0
    for rep in range(4):
        for t in outs:
            t.fill_(-7.0)                     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, r, o in zip(("dx", "dalpha", "dgamma", "dbeta"), ref, outs):
            assert torch.equal(_bits(r), _bits(o)), f"{name} differs (replay {rep})"
