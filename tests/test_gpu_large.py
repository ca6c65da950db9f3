"""More than 2^31 elements (64-bit offsets) on both tile layouts.

Inputs are drawn on the device with a seeded torch generator (17 GB per
case would take minutes to draw on the host). y is checked against the fp64
oracle on sampled elements, including those around element 2^31; with
alpha = +inf and integer dy, dx must be NaN everywhere and dgamma, dbeta,
dalpha are exact integers, checked against int64 sums; a second backward at
alpha = 0.75 checks dx at the same sampled elements."""
import numpy as np
import pytest
import torch

from gpu_util import assert_reports, log, to_np
from oracle import compare, dyt_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dyt():
    import __graft_entry__ as ge
    ge._ensure_built()
    import bwd_dyt_forward_amd as m
    return m


@pytest.mark.parametrize("M,N", [(524291, 4096), ((1 << 26) + 3, 32)])
def test_more_than_2_31_elements(dyt, M, N):
    total = M * N
    assert total > 2 ** 31
    free, _ = torch.cuda.mem_get_info()
    if free < 40 * 2 ** 30:
        pytest.skip("needs ~40 GB of free device memory")
    log(f"[large] M={M} N={N} elements={total} plan={dyt.dyt_get_plan(M, N, 'bf16', 'f32')}")
    g = torch.Generator(device="cuda").manual_seed(M + N)
    x = torch.randn(M, N, generator=g, device="cuda", dtype=torch.bfloat16)
    x.masked_fill_(x == 0, 1.0)
    dy = torch.randint(-3, 4, (M, N), generator=g, device="cuda", dtype=torch.int8).to(torch.bfloat16)
    gamma = torch.rand(N, generator=g, device="cuda") + 0.5
    beta = torch.randn(N, generator=g, device="cuda") * 0.1
    alpha = torch.full((1,), float("inf"), device="cuda")
    y = dyt.dyt_forward(x, alpha, gamma, beta)
    dx, da, dg, db = dyt.dyt_backward(x, dy, alpha, gamma)
    torch.cuda.synchronize()

    # y at sampled elements (random, and around element 2^31 and the end)
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([rng.integers(0, total, 1 << 18),
                                    np.arange(2 ** 31 - 4096, min(2 ** 31 + 4096, total)),
                                    np.arange(total - 4096, total)]))
    assert idx[0] >= 0 and idx[-1] < total
    it = torch.from_numpy(idx).cuda()
    xs = to_np(x.view(-1)[it])
    cols = idx % N
    ys, ss = dyt_oracle.forward_at(xs, cols, [np.inf], to_np(gamma), to_np(beta))
    assert_reports(f"large y M={M} N={N}", [compare.check_y(to_np(y.view(-1)[it]), ys, ss, "bf16")])

    # alpha = +inf with x != 0: dx NaN everywhere, exact integer gradients
    assert bool(torch.isnan(dx).all())
    dyi = dy.to(torch.int8)
    want_db = dyi.sum(dim=0, dtype=torch.int64)
    dyi = torch.where(x < 0, -dyi, dyi)   # dy * sign(x)
    want_dg = dyi.sum(dim=0, dtype=torch.int64)
    del dyi
    assert torch.equal(db.double(), want_db.double())
    assert torch.equal(dg.double(), want_dg.double())
    assert float(da[0]) == 0.0

    # finite alpha: dx at the same sampled elements against the oracle
    del dx
    a2 = torch.full((1,), 0.75, device="cuda")
    dx2, _, _, _ = dyt.dyt_backward(x, dy, a2, gamma)
    torch.cuda.synchronize()
    dys = to_np(dy.view(-1)[it])
    want = dyt_oracle.backward_dx_at(xs, dys, cols, [0.75], to_np(gamma))
    dga = np.abs(dys * to_np(gamma)[cols] * 0.75)
    assert_reports(f"large dx M={M} N={N}",
                   [compare.check_dx(to_np(dx2.view(-1)[it]), want, "bf16", dga)])
    del x, dy, y, dx2
    torch.cuda.empty_cache()
