"""Offline tuner of the DyT tile table (csrc/dyt_tune_table.inc).

The plan of the HIP library is a pure function of the shape: a static table,
keyed by x dtype, row-length range and problem-size range, sets how small packed tiles may get
(min_tiles: the largest K that still yields that many tiles), the largest K
of row segments (kcap) and the forward/backward grid sizes. This script
measures candidate settings and writes the table; the library reads it at
compile time, so results never depend on a run-time measurement (the
Liger-Kernel pull request "fix(dyt): use a 1D grid and tile small-width
rows" autotunes BLOCK_M / BLOCK_N at run time instead).

    python bwd_dyt_forward_amd/tune.py build DIR       # CPU: one library per candidate
    python bwd_dyt_forward_amd/tune.py measure DIR OUT # GPU: time every candidate
    python bwd_dyt_forward_amd/tune.py emit OUT        # write csrc/dyt_tune_table.inc

The measurement record the current table was emitted from is
bwd_dyt_forward_amd/tune_results.json (per shape and candidate, the median
microseconds of the forward, the backward and the residual forward);
tune_results_repeat.json is a second, later run of the same measurement,
kept to show how much the choice moves between runs.
    python bwd_dyt_forward_amd/tune.py defaults        # the table of default constants

Measurement: every candidate library times the forward, the backward (both
passes) and the residual forward of representative shapes per (dtype, range), each sample a run
of back-to-back calls between two events, candidates interleaved over
rounds, medians. The element-wise outputs of every candidate must equal the
default candidate's bit for bit and the gradients must agree to 1e-4
relative; any error or disagreement aborts the run (a failing candidate is
an error, not a loss).

Each table row (dtype, row-length range, size range) has two representative
shapes (the sizes at the range's two ends), and the measured workloads that
fall in it as further representatives. The forward, the backward and the
residual forward each take, among the candidates whose mean time relative to
the default over those shapes is at least 3% better and that are at most 3%
slower at each, the one whose slowest shape (relative to the default) is the
fastest, so that the shapes between them do well too; else the default
(samples of ~10 ms, five interleaved rounds). The residual backward shares the
backward's plan, so that its parameter gradients equal the plain backward's
bit for bit.
"""
from __future__ import annotations

import ctypes
import json
import os
import statistics
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(PKG, "csrc", "dyt_tune_table.inc")

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
DTYPE_NAMES = {0: "DYT_F32", 1: "DYT_BF16", 2: "DYT_F16"}
# row-length ranges of the table and a representative N inside each
RANGES = [(1, 16, 8), (17, 48, 32), (49, 80, 64), (81, 160, 100), (161, 512, 255),
          (513, 2048, 768), (2049, 6144, 4096), (6145, 1 << 30, 8192)]
# problem-size ranges (elements M * N) and their representative sizes
# (2^27: the 32768 x 4096 and 4194304 x 32 workloads at N = 4096, 32)
# Each range is represented by the sizes at its two ends, shared with the
# neighbouring ranges; the top range (2^27 and up, where the 2-byte forward
# prefers smaller tiles by 3-10% while at 2^26 the candidates are within 2%)
# by its lower edge alone.
SIZES = [(1, (1 << 22) - 1, (1 << 20, 1 << 22)), (1 << 22, (1 << 24) - 1, (1 << 22, 1 << 24)),
         (1 << 24, (1 << 26) - 1, (1 << 24, 1 << 26)), (1 << 26, (1 << 27) - 1, (1 << 26, 1 << 27)),
         (1 << 27, 1 << 62, (1 << 27,))]
REP_SIZES = sorted({e for _, _, reps in SIZES for e in reps})
DEFAULT = "a_mt1024_k0_g256"
# name -> (min_tiles, kcap, fwd_grid, bwd_grid); min_tiles acts on packed
# rows and kcap on row segments, so each build serves both kinds of range
CANDIDATES = {
    "a_mt1024_k0_g256": (1024, 0, 256, 256),
    "b_mt4096_k2_g256": (4096, 2, 256, 256),
    "c_mt16384_k1_g256": (16384, 1, 256, 256),
    "d_mt1024_k0_g512": (1024, 0, 512, 512),
    "e_mt4096_k2_g512": (4096, 2, 512, 512),
    "f_mt16384_k1_g512": (16384, 1, 512, 512),
    "g_mt1024_k0_fg1024": (1024, 0, 1024, 256),
    "h_mt4096_k2_fg1024": (4096, 2, 1024, 256),
    "i_mt16384_k1_fg1024": (16384, 1, 1024, 256),
    "j_mt1M_k1_g512": (1 << 20, 1, 512, 512),
    "k_mt1M_k1_fg1024": (1 << 20, 1, 1024, 256),
    # packed rows of 161-512 columns: min tiles 4,096 still gives K = 4 and
    # 16,384 already K = 1; 8,192 reaches K = 2 (half as many rows per tile)
    "l_mt8192_k0_g256": (8192, 0, 256, 256),
}


def _flags(c):
    mt, kc, fg, bg = c
    return ["-DDYT_TUNE_TABLE=0", f"-DDYT_MIN_TILES={mt}", f"-DDYT_WIDE_KCAP={kc}",
            f"-DDYT_FWD_GRID={fg}", f"-DDYT_BWD_GRID={bg}"]


def cmd_build(out_dir: str) -> None:
    sys.path.insert(0, PKG)
    import build
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(out_dir, exist_ok=True)

    def one(name):
        build.build(os.path.join(out_dir, name + ".so"), _flags(CANDIDATES[name]), with_stream_ref=False)
        return name
    with ThreadPoolExecutor(3) as ex:
        for name in ex.map(one, CANDIDATES):
            print("built", name, flush=True)


# The measured workloads (workloads/__init__.py: 1,024 x 64 float32, 65,537 x
# 16 bfloat16, 100,003 x 17 / 100 / 255 float32; 32,768 x 4,096 and
# 4,194,304 x 32 bfloat16 are already range ends) also represent the rows
# they fall in: K follows M through min_tiles, so a shape inside a range can
# get a plan that neither end measured.
WORKLOADS = [("f32", 1024, 64), ("bf16", 65537, 16), ("f32", 100003, 17), ("f32", 100003, 100),
             ("f32", 100003, 255)]


def _range_of(n):
    return next((lo, hi) for lo, hi, _ in RANGES if lo <= n <= hi)


def _shapes():
    """(dtype, n_lo, n_hi, size, M, N, workload) of every measured shape."""
    for d in DTYPES:
        for lo, hi, n in RANGES:
            for e in REP_SIZES:
                yield d, lo, hi, e, max(1, e // n), n, False
    for d, M, N in WORKLOADS:
        lo, hi = _range_of(N)
        yield d, lo, hi, M * N, M, N, True


def cmd_measure(lib_dir: str, out: str, rounds: int = 5, sample_us: float = 10000.0) -> None:
    import torch
    sys.path.insert(0, os.path.dirname(PKG))
    from bwd_dyt_forward_amd import _lib
    libs = {n: _lib._load(os.path.join(lib_dir, n + ".so"), _flags(c)) for n, c in CANDIDATES.items()}
    td = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    s = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    results = []
    for d, lo, hi, e, M, N, wl in _shapes():
        code = DTYPES[d]
        g = torch.Generator(device="cuda").manual_seed(M * 7 + N)
        x = torch.randn(M, N, device="cuda", generator=g).to(td[d])
        dy = torch.randn(M, N, device="cuda", generator=g).to(td[d])
        a = torch.full((1,), 0.5, device="cuda")
        gm = 1 + 0.1 * torch.randn(N, device="cuda", generator=g)
        b = 0.1 * torch.randn(N, device="cuda", generator=g)
        wsb = max(16, max(int(L.dyt_backward_workspace_size(M, N, code, 0)) for L in libs.values()))
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        rres = torch.randn(M, N, device="cuda", generator=g).to(td[d])
        outs = {}
        for name, L in libs.items():
            y, dx = torch.empty_like(x), torch.empty_like(x)
            da, dg, db = torch.empty(1, device="cuda"), torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
            h, y2 = torch.empty_like(x), torch.empty_like(x)
            outs[name] = (y, dx, da, dg, db, h, y2)
        ops = {}
        for name, L in libs.items():
            y, dx, da, dg, db, h, y2 = outs[name]
            ops[(name, "rfwd")] = (lambda L=L, h=h, y2=y2: L.dyt_forward_residual(
                P(x), P(rres), P(a), P(gm), P(b), P(h), P(y2), M, N, code, 0, s))
            ops[(name, "fwd")] = (lambda L=L, y=y: L.dyt_forward(P(x), P(a), P(gm), P(b), P(y), M, N, code, 0, s))
            ops[(name, "bwd")] = (lambda L=L, dx=dx, da=da, dg=dg, db=db: L.dyt_backward(
                P(x), P(dy), P(a), P(gm), P(dx), P(da), P(dg), P(db), P(ws), wsb, M, N, code, 0, s))
        for k, f in ops.items():
            st = f()
            if st != 0:
                raise RuntimeError(f"candidate {k} failed with status {st} on {d} {M}x{N}")
        torch.cuda.synchronize()
        ref = outs[DEFAULT]
        for name, o in outs.items():
            for i in (0, 1, 5, 6):
                if not torch.equal(o[i].view(torch.int16 if o[i].element_size() == 2 else torch.int32),
                                   ref[i].view(torch.int16 if ref[i].element_size() == 2 else torch.int32)):
                    raise RuntimeError(f"candidate {name}: element-wise output {i} differs on {d} {M}x{N}")
            for i in (2, 3, 4):   # normwise: summation orders differ between plans
                err = float((o[i] - ref[i]).abs().max() / ref[i].abs().max().clamp_min(1e-3))
                if not err <= 1e-4:
                    raise RuntimeError(f"candidate {name}: gradient {i} differs by {err:.3g} on {d} {M}x{N}")
        # time: ~10 ms per sample
        t0 = time.perf_counter()
        for _ in range(10):
            ops[(DEFAULT, "bwd")]()
        torch.cuda.synchronize()
        est = (time.perf_counter() - t0) / 10 * 1e6
        reps = int(min(2000, max(10, sample_us / max(est, 1.0))))
        samples = {k: [] for k in ops}
        keys = list(ops)
        for rnd in range(rounds):
            for k in keys[rnd % len(keys):] + keys[:rnd % len(keys)]:
                f = ops[k]
                for _ in range(3):
                    f()
                e0.record()
                for _ in range(reps):
                    f()
                e1.record()
                e1.synchronize()
                samples[k].append(e0.elapsed_time(e1) * 1e3 / reps)
        res = {"dtype": d, "n_lo": lo, "n_hi": hi, "size": e, "M": M, "N": N, "workload": wl,
               "us": {name: {k: statistics.median(samples[(name, k)]) for k in ("fwd", "bwd", "rfwd")}
                      for name in libs}}
        results.append(res)
        best = min(res["us"], key=lambda n: res["us"][n]["fwd"] + res["us"][n]["bwd"])
        print(f"{d:5s} {M:8d} x {N:5d}: default {res['us'][DEFAULT]['fwd']:.1f}/{res['us'][DEFAULT]['bwd']:.1f} us, "
              f"best {best} {res['us'][best]['fwd']:.1f}/{res['us'][best]['bwd']:.1f} us", flush=True)
        del x, dy, rres, ws, outs, ops
        torch.cuda.empty_cache()
    for r in results:    # medians to 0.001 us: the record stays small
        r["us"] = {n: {k: round(v, 3) for k, v in t.items()} for n, t in r["us"].items()}
    with open(out, "w") as f:
        json.dump({"device": torch.cuda.get_device_name(0), "rounds": rounds, "sample_us": sample_us,
                   "candidates": CANDIDATES, "default": DEFAULT, "results": results}, f,
                  separators=(",", ":"))
        f.write("\n")


def _dir(c, fwd: bool) -> str:
    mt, kc, fg, bg = c
    return f"{{{mt}, {kc}, {fg if fwd else bg}}}"


def _entry(dt, lo, hi, e_lo, e_hi, cf, cb, cr, note):
    return (f"    {{{DTYPE_NAMES[dt]}, {lo}, {hi}, {e_lo}, {e_hi}, {_dir(cf, True)}, "
            f"{_dir(cb, False)}, {_dir(cr, True)}}},  // {note}")


HEADER = ["// dyt_tune_table.inc - generated by bwd_dyt_forward_amd/tune.py; do not edit by hand.",
          "// {x dtype, N from, N to, M*N from, M*N to, forward {min_tiles, kcap, grid},",
          "//  backward {min_tiles, kcap, grid}, residual forward {min_tiles, kcap, grid}}"]
ADOPT = 0.97      # a candidate replaces the default only if at least 3% faster


GUARD = 1.03      # ... and at most 3% slower at any representative of its range


def _choose(reps, cands, dflt, key):
    """Among the candidates at least 3% faster than the default on the mean
    time ratio over the range's representatives and at most 3% slower at
    each, the one whose slower representative is the fastest (the shapes
    between a range's two ends should do well at both); else the default."""
    ratios = {n: [q["us"][n][key] / q["us"][dflt][key] for q in reps] for n in cands}
    ok = [n for n, v in ratios.items() if max(v) <= GUARD and statistics.fmean(v) <= ADOPT]
    if not ok:
        return dflt, ratios[dflt]
    best = min(ok, key=lambda n: (max(ratios[n]), statistics.fmean(ratios[n])))
    return best, ratios[best]


def emit_text(path: str) -> str:
    """The table (dyt_tune_table.inc) that the measurement record at path gives."""
    with open(path) as f:
        data = json.load(f)
    cands = {k: tuple(v) for k, v in data["candidates"].items()}
    dflt = data["default"]
    last = chr(ord("a") + len(cands) - 1)
    lines = HEADER + ["// measured with tune.py measure on one MI355X (interleaved rounds, medians; "
                      f"record: bwd_dyt_forward_amd/{os.path.basename(path)}); "
                      f"note = representative shapes, chosen candidate (a-{last}, see tune.py) and its times "
                      "relative to the default a (forward; backward; residual forward)"]
    groups = {}
    for d in DTYPES:
        for lo, hi, _ in RANGES:
            for e_lo, e_hi, sizes in SIZES:
                groups[(d, lo, hi, e_lo, e_hi)] = [
                    r for r in data["results"]
                    if r["dtype"] == d and r["n_lo"] == lo
                    and (r["size"] in sizes if not r.get("workload") else e_lo <= r["size"] <= e_hi)]
    for (d, lo, hi, e_lo, e_hi), reps in groups.items():
        picks = [_choose(reps, cands, dflt, k) for k in ("fwd", "bwd", "rfwd")]
        note = (" ".join(f"{q['M']}x{q['N']}" for q in reps) + ": "
                + "; ".join(f"{b[0]} " + "/".join(f"{v:.3f}" for v in rt) for b, rt in picks))
        lines.append(_entry(DTYPES[d], lo, hi, e_lo, e_hi, cands[picks[0][0]], cands[picks[1][0]],
                            cands[picks[2][0]], note))
    return "\n".join(lines) + "\n"


def cmd_emit(path: str) -> None:
    text = emit_text(path)
    with open(TABLE, "w") as f:
        f.write(text)
    print(text, end="")


def cmd_defaults() -> None:
    lines = HEADER + ["// defaults (no measurement)"]
    c = CANDIDATES[DEFAULT]
    for d, code in DTYPES.items():
        for lo, hi, _ in RANGES:
            for e_lo, e_hi, _ in SIZES:
                lines.append(_entry(code, lo, hi, e_lo, e_hi, c, c, c, "default"))
    with open(TABLE, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    cmd = sys.argv[1] if len(sys.argv) > 1 else ""
    if cmd == "build" and len(sys.argv) == 3:
        cmd_build(sys.argv[2])
    elif cmd == "measure" and len(sys.argv) == 4:
        cmd_measure(sys.argv[2], sys.argv[3])
    elif cmd == "emit" and len(sys.argv) == 3:
        cmd_emit(sys.argv[2])
    elif cmd == "defaults":
        cmd_defaults()
    else:
        print(__doc__)
        sys.exit(2)
