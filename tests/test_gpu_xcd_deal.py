"""The forward's XCD-weighted deal under both parities. Tiles of one vector
slot are dealt with the larger share to the workgroups expected on the even
XCDs: even workgroup indices, or odd ones when the launch's flip is 1 (the
hardware starts some queues on an odd XCD). Every tile must be computed
exactly once either way, so y is bit-identical under flip 0, flip 1 and the
recorded hint, with y pre-filled with a canary that no output equals; y is
also checked against the fp64 oracle on sampled elements. A weighted launch
records the XCD its first workgroup ran on (dyt_xcd_hint)."""
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
    yield m
    m.dyt_set_xcd_flip_override(-1)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy().copy()


# (M, N, x dtype, param dtype): tiled forwards of one vector slot with at
# least 8 tiles per workgroup (the weighted deal; asserted from the plan)
SHAPES = [
    (16384, 4096, "bf16", "f32"),     # row segments, two per row, 1,024 workgroups
    (100003, 255, "f32", "f32"),      # packed rows, float32 (sc1 stores), partial tile
    (32771, 4096, "f16", "bf16"),     # rows left over after the last whole group
    (21848, 6144, "bf16", "f32"),     # three segments per row, 510 workgroups
    (300007, 64, "f32", "f32"),       # packed rows of 16
]


@pytest.mark.parametrize("M,N,xdt,pdt", SHAPES)
def test_weighted_deal_is_exact_under_both_parities(dyt, M, N, xdt, pdt):
    log(f"[xcd deal] {M}x{N} {xdt}/{pdt}")
    plan = dyt.dyt_get_forward_plan(M, N, xdt, pdt)
    assert plan["flat"] == 0 and plan["slots"] == 1 and plan["vec"] > 1
    assert plan["tiles"] >= 8 * plan["fwd_grid"] and plan["fwd_grid"] % (2 * plan["col_blocks"]) == 0
    inp = workloads.custom(M, N, xdt, pdt, seed=M % 97)
    x = torch.from_numpy(inp.x).cuda().to(TORCH_DT[xdt])
    a, g, b = (torch.from_numpy(v).cuda().to(TORCH_DT[pdt]) for v in (inp.alpha, inp.gamma, inp.beta))
    outs = {}
    for flip in (0, 1, -1):
        dyt.dyt_set_xcd_flip_override(flip)
        y = torch.full_like(x, float("nan"))
        dyt.dyt_forward(x, a, g, b, y=y)
        torch.cuda.synchronize()
        outs[flip] = y
    dyt.dyt_set_xcd_flip_override(-1)
    b0 = _bits(outs[0])
    assert not torch.isnan(outs[0]).any(), "a tile was not computed under flip 0"
    assert np.array_equal(b0, _bits(outs[1])), "flip 1 differs from flip 0"
    assert np.array_equal(b0, _bits(outs[-1])), "the hinted launch differs from flip 0"
    hint = dyt.dyt_xcd_hint()
    log(f"  recorded XCD of workgroup 0: {hint}")
    assert 0 <= hint < 8
    # against the oracle at sampled elements
    total = M * N
    rng = np.random.default_rng(7)
    idx = np.unique(np.concatenate([rng.integers(0, total, size=min(1 << 18, total)),
                                    np.arange(min(4096, total)), np.arange(max(0, total - 4096), total)]))
    rows, cols = np.divmod(idx, N)
    ys, ss = dyt_oracle.forward_at(inp.x[rows, cols], cols, inp.alpha, inp.gamma, inp.beta)
    y_g = to_np(outs[0].reshape(-1)[torch.from_numpy(idx).cuda()])
    assert_reports(f"{M}x{N}", [compare.check_y(y_g, ys, ss, xdt, "y[sampled]")])
