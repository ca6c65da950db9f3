"""Helpers shared by the GPU tests: upload workload inputs, run the HIP path
through the C ABI binding, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import compare, dyt_oracle

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def upload(inp, dev="cuda"):
    xdt, pdt = TORCH_DT[inp.x_dtype], TORCH_DT[inp.p_dtype]
    return dict(
        x=torch.from_numpy(inp.x).to(dev).to(xdt),
        dy=torch.from_numpy(inp.dy).to(dev).to(xdt),
        alpha=torch.from_numpy(inp.alpha).to(dev).to(pdt),
        gamma=torch.from_numpy(inp.gamma).to(dev).to(pdt),
        beta=torch.from_numpy(inp.beta).to(dev).to(pdt),
    )


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_both(dyt, d):
    y = dyt.dyt_forward(d["x"], d["alpha"], d["gamma"], d["beta"])
    dx, da, dg, db = dyt.dyt_backward(d["x"], d["dy"], d["alpha"], d["gamma"])
    torch.cuda.synchronize()
    return y, dx, da, dg, db


def full_reports(inp, y, dx, da, dg, db):
    """Element-by-element comparison of every output with the full oracle."""
    f = dyt_oracle.forward(inp.x, inp.alpha, inp.gamma, inp.beta)
    r = dyt_oracle.backward(inp.x, inp.dy, inp.alpha, inp.gamma)
    dga = np.abs(inp.dy.astype(np.float64) * inp.gamma.astype(np.float64) * float(inp.alpha[0]))
    return [
        compare.check_y(to_np(y), f.y, f.scale, inp.x_dtype),
        compare.check_dx(to_np(dx), r.dx, inp.x_dtype, dga),
        compare.check_grad(to_np(dg), r.dgamma, r.rss_dgamma, inp.p_dtype, "dgamma"),
        compare.check_grad(to_np(db), r.dbeta, r.rss_dbeta, inp.p_dtype, "dbeta"),
        compare.check_grad(to_np(da), r.dalpha, r.rss_dalpha, inp.p_dtype, "dalpha"),
    ]


def sampled_reports(inp, y, dx, da, dg, db, n_random=1 << 20, seed=123):
    """Large inputs: y and dx at sampled positions (random + first and last
    4096 elements) computed one by one; grads against the full-sum oracle."""
    M, N = inp.x.shape
    total = M * N
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([
        rng.integers(0, total, size=min(n_random, total)),
        np.arange(min(4096, total)), np.arange(max(0, total - 4096), total)]))
    rows, cols = np.divmod(idx, N)
    xs = inp.x[rows, cols]
    dys = inp.dy[rows, cols]
    ys, ss = dyt_oracle.forward_at(xs, cols, inp.alpha, inp.gamma, inp.beta)
    dxs = dyt_oracle.backward_dx_at(xs, dys, cols, inp.alpha, inp.gamma)
    idx_t = torch.from_numpy(idx).to(y.device)
    y_g = to_np(y.reshape(-1)[idx_t])
    dx_g = to_np(dx.reshape(-1)[idx_t])
    r = dyt_oracle.backward(inp.x, inp.dy, inp.alpha, inp.gamma, want_dx=False)
    dga = np.abs(dys.astype(np.float64) * inp.gamma[cols].astype(np.float64) * float(inp.alpha[0]))
    return [
        compare.check_y(y_g, ys, ss, inp.x_dtype, "y[sampled]"),
        compare.check_dx(dx_g, dxs, inp.x_dtype, dga, "dx[sampled]"),
        compare.check_grad(to_np(dg), r.dgamma, r.rss_dgamma, inp.p_dtype, "dgamma"),
        compare.check_grad(to_np(db), r.dbeta, r.rss_dbeta, inp.p_dtype, "dbeta"),
        compare.check_grad(to_np(da), r.dalpha, r.rss_dalpha, inp.p_dtype, "dalpha"),
    ]


def assert_reports(tag, reps):
    for rep in reps:
        log(f"  {tag}: {rep}")
    bad = [str(rep) for rep in reps if not rep.ok]
    assert not bad, f"{tag}: " + "; ".join(bad)


def merge_reports(name, parts):
    """One report over the concatenation of chunk reports: parts is a list of
    (element offset of the chunk, Report)."""
    out = compare.Report(name, 0)
    for off, rep in parts:
        out.n += rep.n
        out.n_fail += rep.n_fail
        out.nan_mismatch += rep.nan_mismatch
        out.inf_mismatch += rep.inf_mismatch
        out.worst_ratio = max(out.worst_ratio, rep.worst_ratio)
        if len(out.first_fail) < 5:
            out.first_fail += [off + i for i in rep.first_fail][:5 - len(out.first_fail)]
    return out


def every_element_reports(inp, y, dx, da, dg, db, rows_per_chunk=None, threads=16):
    """Every element of y and dx against the oracle, in row chunks on host
    threads (NumPy releases the interpreter lock inside its array loops);
    the gradients against the sums of the same chunks' oracle results."""
    from concurrent.futures import ThreadPoolExecutor
    M, N = inp.x.shape
    rows = rows_per_chunk or max(1, (1 << 21) // N)
    y_h = y.float().cpu().numpy()
    dx_h = dx.float().cpu().numpy()
    cols = np.arange(N)
    dga_col = np.abs(inp.gamma.astype(np.float64) * float(inp.alpha[0]))

    def work(r0):
        r1 = min(M, r0 + rows)
        xc, dyc = inp.x[r0:r1], inp.dy[r0:r1]
        yo, so = dyt_oracle.forward_at(xc, cols, inp.alpha, inp.gamma, inp.beta)
        b = dyt_oracle.backward(xc, dyc, inp.alpha, inp.gamma)
        ry = compare.check_y(y_h[r0:r1], yo, so, inp.x_dtype, "y")
        rdx = compare.check_dx(dx_h[r0:r1], b.dx, inp.x_dtype, np.abs(dyc.astype(np.float64)) * dga_col, "dx")
        sums = (b.dgamma, b.dbeta, b.dalpha, b.rss_dgamma ** 2, b.rss_dbeta ** 2, b.rss_dalpha ** 2)
        return r0 * N, ry, rdx, sums

    with ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(work, range(0, M, rows)))
    dgo = sum(r[3][0] for r in res)
    dbo = sum(r[3][1] for r in res)
    dao = sum(r[3][2] for r in res)
    rss = [np.sqrt(sum(r[3][k] for r in res)) for k in (3, 4, 5)]
    return [
        merge_reports("y[every element]", [(r[0], r[1]) for r in res]),
        merge_reports("dx[every element]", [(r[0], r[2]) for r in res]),
        compare.check_grad(to_np(dg), dgo, rss[0], inp.p_dtype, "dgamma"),
        compare.check_grad(to_np(db), dbo, rss[1], inp.p_dtype, "dbeta"),
        compare.check_grad(to_np(da), dao, rss[2], inp.p_dtype, "dalpha"),
    ]
