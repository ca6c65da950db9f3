#!/usr/bin/env python3
"""Benchmark of the fused DyT layer on one MI355X: one step = forward +
backward (both passes) over one batch of synthetic input resident in HBM.

Prints ONE JSON line on stdout:
  value        whole-step effective HBM throughput (GB/s) = algorithmic bytes
               of forward + backward / measured step time
  roofline     the dominant kernel (backward pass 1) against the 8 TB/s HBM
               peak: algorithmic bytes per launch / mean launch duration from
               HIP events recorded on the launch stream around a timed run of
               back-to-back launches
  cpu_baseline the fp64 CPU oracle timed on a bounded sample of the same
               workload, on one pinned host core
  stream_ceiling  measured ceilings on the same tensor size: a plain 16-byte
               copy and a 2-in/1-out stream (reference kernels in
               libdyt_streamref.so), with the forward's and pass 1's fraction
               of them
Algorithmic bytes (sx = x dtype size, sp = parameter dtype size):
  forward   2 M N sx + (2N + 1) sp      backward 3 M N sx + (3N + 2) sp
  pass 1    3 M N sx + (N + 1) sp       pass 2   (2N + 1) sp
(workspace traffic of the backward is excluded from the algorithmic bytes).

With the residual add fused in front (h = x + r, y = DyT(h); backward
dh = dres + dx), the line also carries "residual": fused and unfused
(torch.add beside the plain layer) times on the same shape.

Timing: W warm-up steps (extended by untimed steps until 0.3 s have passed,
because the GPU clocks ramp for the first ~100 steps after idle), then timed
regions, each bracketed by one pair of HIP events on the launch stream and
entered with one untimed call already queued: A, K whole steps (the reported
value and ms_per_step); B, K back-to-back launches of backward pass 1 (the
roofline figure); C, K back-to-back forwards; D, K back-to-back backwards
(pass 1 + pass 2; pass 2's share is D - B). B, C and D are medians of three
runs. No event is recorded between two kernels of a timed run: on some
MI355X boxes each such record adds several microseconds to the kernel it
brackets (events around every kernel of a step have read the 32,768 x 4,096
forward at 91-93 us whose kernel trace shows 79.5 us).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "c4_32768x4096_bf16"        # the transformer-block shape the 80% target names
SECONDARY = "c5_4194304x32_bf16_outliers"  # the narrow-row bulk shape the 60% target names
HBM_PEAK_GBPS = 8000.0                 # MI355X HBM3E, vendor figure
SETTLE_S = 0.3                         # minimum untimed warm-up wall time
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _build_module():
    """bwd_dyt_forward_amd/build.py, loaded by path (no torch, no library)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_dyt_build", os.path.join(ROOT, "bwd_dyt_forward_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def kernel_source_hash() -> str:
    """Build id of the current sources (hash of the kernel, launch and host
    sources without comments, and of the compiler flags), so that counter
    figures stay attached to the code they measured."""
    return _build_module().source_hash()


def algorithmic_bytes(M: int, N: int, sx: int, sp: int) -> dict:
    return {
        "fwd": 2 * M * N * sx + (2 * N + 1) * sp,
        "bwd": 3 * M * N * sx + (3 * N + 2) * sp,
        "pass1": 3 * M * N * sx + (N + 1) * sp,
        "pass2": (2 * N + 1) * sp,
    }


def graph_step_us(dyt, torch, x, dy, a, g, b, y, dx, ws, da, dg, db, M, N, xdt, reps: int = 50) -> float:
    """One step (forward, pass 1, pass 2) captured in a HIP graph and, after
    a settling run of replays, replayed `reps` times back to back: the
    per-step time without host launch cost."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):     # warm up on the capture stream
            dyt.dyt_forward(x, a, g, b, y=y)
            dyt.dyt_backward_partials(x, dy, a, g, dx, ws)
            dyt.dyt_backward_finish(ws, M, N, xdt, da, dg, db)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dyt.dyt_forward(x, a, g, b, y=y)
        dyt.dyt_backward_partials(x, dy, a, g, dx, ws)
        dyt.dyt_backward_finish(ws, M, N, xdt, da, dg, db)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:   # settle the clocks on replays
        for _ in range(10):
            graph.replay()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def cold_times(dyt, torch, x, dy, a, g, b, y, dx, ws, da, dg, db, M, N, xdt, iters, B) -> dict:
    """Cold-cache timing: before each timed launch a 1 GiB buffer is read
    (four times the 256 MB MALL, far above the L2s), then HIP events bracket
    the forward, and after another flush the backward (pass 1 + pass 2).
    The flush only reads, so it leaves clean lines: a flush that writes
    leaves the caches full of dirty lines whose write-back the timed kernel
    would pay for. Median, 10th and 90th percentile over `iters` repetitions
    (microseconds)."""
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    sink = torch.empty((), dtype=torch.int64, device="cuda")
    fwd, bwd = [], []
    for i in range(iters + 3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.sum(flush, dim=0, dtype=torch.int64, out=sink)
        ev[0].record()
        dyt.dyt_forward(x, a, g, b, y=y)
        ev[1].record()
        torch.sum(flush, dim=0, dtype=torch.int64, out=sink)
        ev[2].record()
        dyt.dyt_backward_partials(x, dy, a, g, dx, ws)
        dyt.dyt_backward_finish(ws, M, N, xdt, da, dg, db)
        ev[3].record()
        ev[3].synchronize()
        if i >= 3:          # the first repetitions warm the code paths
            fwd.append(ev[0].elapsed_time(ev[1]) * 1e3)
            bwd.append(ev[2].elapsed_time(ev[3]) * 1e3)
    del flush
    torch.cuda.empty_cache()

    def q(v, f):
        v = sorted(v)
        return v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
    out = {}
    for k, v, nb in (("fwd", fwd, B["fwd"]), ("bwd", bwd, B["bwd"])):
        med = statistics.median(v)
        out[k] = {"p50_us": med, "p10_us": q(v, 0.1), "p90_us": q(v, 0.9),
                  "gbps": nb / (med * 1e-6) / 1e9}
    return out


def measure(dyt, torch, name: str, steps: int, warmup: int, graph: bool = False,
            cold_iters: int = 0) -> dict:
    import workloads
    cfg = workloads.CONFIGS[name]
    t0 = time.perf_counter()
    inp = workloads.generate(name)
    log(f"[bench] {name}: inputs drawn in {time.perf_counter() - t0:.1f}s")
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    xdt, pdt = tdt[inp.x_dtype], tdt[inp.p_dtype]
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp.x).to(dev).to(xdt)
    dy = torch.from_numpy(inp.dy).to(dev).to(xdt)
    a = torch.from_numpy(inp.alpha).to(dev).to(pdt)
    g = torch.from_numpy(inp.gamma).to(dev).to(pdt)
    b = torch.from_numpy(inp.beta).to(dev).to(pdt)
    del inp
    M, N = cfg.M, cfg.N
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    dg = torch.empty(N, dtype=pdt, device=dev)
    db = torch.empty(N, dtype=pdt, device=dev)
    da = torch.empty(1, dtype=pdt, device=dev)
    need = dyt.dyt_backward_workspace_size(M, N, xdt, pdt)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        dyt.dyt_forward(x, a, g, b, y=y, stream=stream)

    def pass1():
        dyt.dyt_backward_partials(x, dy, a, g, dx, ws, stream=stream)

    def bwd():
        pass1()
        dyt.dyt_backward_finish(ws, M, N, xdt, da, dg, db, stream=stream)

    def step():
        fwd()
        bwd()

    def run_us(fn, n, rounds=3):
        """Microseconds per call of n back-to-back calls of fn between one
        pair of HIP events on the launch stream, entered with one untimed
        call queued (the GPU is busy while the host records the first
        event); median over rounds."""
        out = []
        for _ in range(rounds):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            fn()
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3 / n)
        return statistics.median(out)

    # Warm-up: `warmup` steps, extended by untimed steps until SETTLE_S of
    # wall time has passed. On MI355X the first ~100 steps after idle run up
    # to 1.6x slower while the clocks ramp; 0.3 s is several times that.
    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - t0 < SETTLE_S:
        step()
        n_warm += 1
        if n_warm % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # Timed region A (the reported value): `steps` whole steps, no events
    # inside.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    step()
    h0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    total_ms = start.elapsed_time(end)

    # Timed regions B, C, D: backward pass 1 (the dominant kernel: the
    # roofline figure), the forward and the backward, each run back to back.
    p1_us = run_us(pass1, steps)
    fwd_us = run_us(fwd, steps)
    bwd_us = run_us(bwd, steps)
    sx = x.element_size()
    sp = a.element_size()
    B = algorithmic_bytes(M, N, sx, sp)
    ms_step = total_ms / steps
    res = {
        "workload": name, "M": M, "N": N, "x_dtype": cfg.x_dtype, "param_dtype": cfg.p_dtype,
        "ms_per_step": ms_step, "host_s": host_s, "warmup_steps_run": n_warm,
        "gbps_step": (B["fwd"] + B["bwd"]) / (ms_step * 1e-3) / 1e9,
        "fwd_us": fwd_us,
        "bwd_us": bwd_us,
        "pass1_us": p1_us,
        "pass2_us": bwd_us - p1_us,
        "fwd_gbps": B["fwd"] / (fwd_us * 1e-6) / 1e9,
        "bwd_gbps": B["bwd"] / (bwd_us * 1e-6) / 1e9,
        "pass1_gbps": B["pass1"] / (p1_us * 1e-6) / 1e9,
        "bytes": B,
        "workspace_bytes": need,
        "plan": dyt.dyt_get_plan(M, N, xdt, pdt, True),
        "fwd_plan": dyt.dyt_get_forward_plan(M, N, xdt, pdt, True),
    }
    res["fwd_frac"] = res["fwd_gbps"] / HBM_PEAK_GBPS
    res["bwd_frac"] = res["bwd_gbps"] / HBM_PEAK_GBPS
    if cold_iters:
        res["cold"] = cold_times(dyt, torch, x, dy, a, g, b, y, dx, ws, da, dg, db, M, N, xdt,
                                 cold_iters, B)
    if graph:
        gus = graph_step_us(dyt, torch, x, dy, a, g, b, y, dx, ws, da, dg, db, M, N, xdt)
        res["graph_step_us"] = gus
        res["graph_step_gbps"] = (B["fwd"] + B["bwd"]) / (gus * 1e-6) / 1e9
    del x, dy, y, dx, ws
    torch.cuda.empty_cache()
    return res


def measure_residual(dyt, torch, name: str, reps: int = 40, rounds: int = 3) -> dict:
    """The residual-fused layer against the same work unfused, on the
    workload's shape: forward h = x + r, y = DyT(h) (fused: one kernel;
    unfused: torch.add then dyt_forward) and backward dh = dres + dx (fused:
    dyt_backward_residual; unfused: dyt_backward then torch.add). Each sample
    is `reps` back-to-back calls between two events (no events inside);
    medians over `rounds` interleaved rounds. Inputs are drawn on the device
    from a seeded generator (N(0, 1) in the workload's x dtype)."""
    import workloads
    cfg = workloads.CONFIGS[name]
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    xdt, pdt = tdt[cfg.x_dtype], tdt[cfg.p_dtype]
    M, N = cfg.M, cfg.N
    gen = torch.Generator(device="cuda").manual_seed(2024)
    mk = lambda: torch.randn(M, N, device="cuda", generator=gen).to(xdt)
    x, r, dy, dres = mk(), mk(), mk(), mk()
    h, y, dh = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    a = torch.full((1,), 0.5, device="cuda").to(pdt)
    g = (1 + 0.02 * torch.randn(N, device="cuda", generator=gen)).to(pdt)
    b = torch.zeros(N, device="cuda").to(pdt)
    da, dg, db = torch.empty_like(a), torch.empty_like(g), torch.empty_like(b)
    ws = torch.empty(max(16, dyt.dyt_backward_workspace_size(M, N, xdt, pdt)), dtype=torch.uint8,
                     device="cuda")
    ops = {
        "fwd_fused": lambda: dyt.dyt_forward_residual(x, r, a, g, b, h=h, y=y),
        "fwd_unfused": lambda: (torch.add(x, r, out=h), dyt.dyt_forward(h, a, g, b, y=y)),
        "bwd_fused": lambda: dyt.dyt_backward_residual(h, dy, dres, a, g, dh=dh, dalpha=da, dgamma=dg,
                                                       dbeta=db, workspace=ws),
        "bwd_unfused": lambda: (dyt.dyt_backward(h, dy, a, g, dx=dh, dalpha=da, dgamma=dg, dbeta=db,
                                                 workspace=ws), torch.add(dh, dres, out=dh)),
    }
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(20):
            ops["fwd_fused"]()
        torch.cuda.synchronize()
    samples = {k: [] for k in ops}
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for _ in range(rounds):
        for k, f in ops.items():
            for _ in range(5):
                f()
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            e1.synchronize()
            samples[k].append(e0.elapsed_time(e1) * 1e3 / reps)
    us = {k: statistics.median(v) for k, v in samples.items()}
    sx, sp = x.element_size(), a.element_size()
    fwd_bytes = 4 * M * N * sx + (2 * N + 1) * sp          # read x, r; write h, y
    bwd_bytes = 4 * M * N * sx + (3 * N + 2) * sp          # read h, dy, dres; write dh
    del x, r, dy, dres, h, y, dh, ws
    torch.cuda.empty_cache()
    return {
        "workload": name,
        "unfused": "torch.add then dyt_forward; dyt_backward then torch.add",
        "fwd": {"fused_us": round(us["fwd_fused"], 2), "unfused_us": round(us["fwd_unfused"], 2),
                "speedup": round(us["fwd_unfused"] / us["fwd_fused"], 3),
                "fused_GBps": round(fwd_bytes / (us["fwd_fused"] * 1e-6) / 1e9, 1)},
        "bwd": {"fused_us": round(us["bwd_fused"], 2), "unfused_us": round(us["bwd_unfused"], 2),
                "speedup": round(us["bwd_unfused"] / us["bwd_fused"], 3),
                "fused_GBps": round(bwd_bytes / (us["bwd_fused"] * 1e-6) / 1e9, 1)},
    }


def stream_ceilings(torch, nbytes: int, reps: int = 40, rounds: int = 3) -> dict:
    """Measured streaming ceilings on tensors of nbytes each, from the
    reference kernels in libdyt_streamref.so (16-byte streams with their
    best measured launch shapes and store kinds): a copy (the forward's 1
    read + 1 write) and a 2-in/1-out stream (backward pass 1's traffic). GB/s count
    every byte read and written; medians of `rounds` samples of `reps`
    back-to-back launches after a settling warm-up."""
    import ctypes
    sys.path.insert(0, os.path.join(ROOT, "bwd_dyt_forward_amd"))
    import build as dyt_build
    lib = ctypes.CDLL(dyt_build.STREAM_REF_PATH, mode=ctypes.RTLD_LOCAL)
    lib.stream_ref_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.stream_ref_2in1out.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_void_p]
    nbytes -= nbytes % 16
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    c = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    ops = {"copy": lambda: lib.stream_ref_copy(a.data_ptr(), c.data_ptr(), nbytes, s),
           "2in1out": lambda: lib.stream_ref_2in1out(a.data_ptr(), b.data_ptr(), c.data_ptr(), nbytes, s)}
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(20):
            if ops["copy"]() != 0:
                raise RuntimeError("stream_ref_copy rejected its arguments")
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    us = {k: [] for k in ops}
    for _ in range(rounds):
        for k, f in ops.items():
            if f() != 0:
                raise RuntimeError(f"stream_ref {k} failed")
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            e1.synchronize()
            us[k].append(e0.elapsed_time(e1) * 1e3 / reps)
    del a, b, c
    torch.cuda.empty_cache()
    return {"copy_GBps": round(2 * nbytes / (statistics.median(us["copy"]) * 1e-6) / 1e9, 1),
            "two_in_one_out_GBps": round(3 * nbytes / (statistics.median(us["2in1out"]) * 1e-6) / 1e9, 1),
            "tensor_bytes": nbytes}


def residual_stream_ceilings(torch, nbytes: int, reps: int = 20, rounds: int = 3) -> dict:
    """The streams of the residual-fused layer on tensors of nbytes each
    (libdyt_streamref.so): two inputs and two outputs (the fused forward's
    traffic) and three inputs and one output (the fused pass 1's), each with
    nontemporal and with write-back stores; GB/s of the faster store kind,
    counting every byte read and written; medians of `rounds` samples of
    `reps` back-to-back launches after a settling run."""
    import ctypes
    sys.path.insert(0, os.path.join(ROOT, "bwd_dyt_forward_amd"))
    import build as dyt_build
    lib = ctypes.CDLL(dyt_build.STREAM_REF_PATH, mode=ctypes.RTLD_LOCAL)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.stream_ref_2in2out.argtypes = [vp, vp, vp, vp, i64, i32, vp]
    lib.stream_ref_3in1out.argtypes = [vp, vp, vp, vp, i64, i32, vp]
    nbytes -= nbytes % 16
    t = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(3)]
    o = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    s = torch.cuda.current_stream().cuda_stream
    p = [x.data_ptr() for x in t] + [x.data_ptr() for x in o]
    ops = {}
    for nt in (0, 1):
        ops[("2in2out", nt)] = (lambda nt=nt: lib.stream_ref_2in2out(p[0], p[1], p[3], p[4], nbytes, nt, s), 4)
        ops[("3in1out", nt)] = (lambda nt=nt: lib.stream_ref_3in1out(p[0], p[1], p[2], p[3], nbytes, nt, s), 4)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for f, _ in ops.values():
            if f() != 0:
                raise RuntimeError("a residual reference stream rejected its arguments")
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    us = {k: [] for k in ops}
    for _ in range(rounds):
        for k, (f, _) in ops.items():
            f()
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            e1.synchronize()
            us[k].append(e0.elapsed_time(e1) * 1e3 / reps)
    del t, o
    torch.cuda.empty_cache()
    out = {"tensor_bytes": nbytes}
    for kind in ("2in2out", "3in1out"):
        best = min((statistics.median(us[(kind, nt)]), nt) for nt in (0, 1))
        out[f"{kind}_GBps"] = round(4 * nbytes / (best[0] * 1e-6) / 1e9, 1)
        out[f"{kind}_stores"] = "nontemporal" if best[1] else "write-back"
    return out


def copy_calibration(torch, mib: int) -> None:
    """A plain elementwise kernel of known size (reads and writes mib MiB each)
    so that HBM byte counters can be scaled; used only by counter runs."""
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {mib} MiB read + {mib} MiB written per launch")


def copy_ceiling(torch, nbytes: int, reps: int = 20) -> float:
    """Device-to-device copy of nbytes (read nbytes + write nbytes) with the
    runtime's copy path, as a measured ceiling for streaming kernels (GB/s,
    counting read + write bytes, median of reps)."""
    n = nbytes // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (statistics.median(times) * 1e-3) / 1e9


def cpu_baseline(name: str, seconds: float) -> dict:
    """The fp64 oracle, as it is, on whole rows of the workload until about
    `seconds` of CPU time, pinned to one core (numpy ufuncs are single-threaded)."""
    import workloads
    from oracle import dyt_oracle
    cfg = workloads.CONFIGS[name]
    rows = max(1, (1 << 20) // cfg.N)          # ~1M elements per chunk
    inp = workloads.generate(name, M=rows)
    sx = 4 if cfg.x_dtype == "f32" else 2
    sp = 4 if cfg.p_dtype == "f32" else 2
    old = os.sched_getaffinity(0)
    core = min(old)
    os.sched_setaffinity(0, {core})
    try:
        done = 0
        t0 = time.perf_counter()
        while True:
            dyt_oracle.forward(inp.x, inp.alpha, inp.gamma, inp.beta)
            dyt_oracle.backward(inp.x, inp.dy, inp.alpha, inp.gamma)
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        os.sched_setaffinity(0, old)
    B = algorithmic_bytes(rows, cfg.N, sx, sp)
    gbps = done * (B["fwd"] + B["bwd"]) / el / 1e9
    return {"value": gbps, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} x ({rows} rows x {cfg.N}) of {name}, forward+backward in fp64, "
                      f"{el:.1f}s on 1 pinned core"}


def oracle_times(name: str, max_elems: int = 1 << 20, runs: int = 3) -> dict:
    """The fp64 oracle, as it is, per direction on a bounded sample of the
    workload (whole rows, at most max_elems elements), pinned to one host
    core; median of `runs` runs, GB/s of the sample's algorithmic bytes."""
    import workloads
    from oracle import dyt_oracle
    cfg = workloads.CONFIGS[name]
    rows = min(cfg.M, max(1, max_elems // cfg.N))
    inp = workloads.generate(name, M=rows)
    sx = 4 if cfg.x_dtype == "f32" else 2
    sp = 4 if cfg.p_dtype == "f32" else 2
    B = algorithmic_bytes(rows, cfg.N, sx, sp)
    old = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(old)})
    try:
        tf, tb = [], []
        for _ in range(runs):
            t0 = time.perf_counter()
            dyt_oracle.forward(inp.x, inp.alpha, inp.gamma, inp.beta)
            tf.append(time.perf_counter() - t0)
            t0 = time.perf_counter()
            dyt_oracle.backward(inp.x, inp.dy, inp.alpha, inp.gamma)
            tb.append(time.perf_counter() - t0)
    finally:
        os.sched_setaffinity(0, old)
    return {"rows": rows, "fwd_gbps": B["fwd"] / statistics.median(tf) / 1e9,
            "bwd_gbps": B["bwd"] / statistics.median(tb) / 1e9}


def host_description() -> str:
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return (f"{model}; os.cpu_count() = {os.cpu_count()}, "
            f"affinity = {len(os.sched_getaffinity(0))} cores; oracle runs pinned to 1 core")


def report_all(dyt, torch, path: str, steps: int = 20, warmup: int = 5) -> None:
    """Every workload shape: steady-state forward / backward times (HIP events,
    means over `steps` continuous steps after `warmup`), written as Markdown."""
    import workloads
    floor_x = torch.zeros(1, 8, dtype=torch.float32, device="cuda")
    floor_p = torch.ones(8, device="cuda")
    a1 = torch.ones(1, device="cuda")
    y1 = torch.empty_like(floor_x)
    for _ in range(20):
        dyt.dyt_forward(floor_x, a1, floor_p, floor_p, y=y1)
    torch.cuda.synchronize()
    fl = []
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(100):       # back-to-back: the queue runs ahead of the host
            dyt.dyt_forward(floor_x, a1, floor_p, floor_p, y=y1)
        e1.record()
        e1.synchronize()
        fl.append(e0.elapsed_time(e1) * 1e3 / 100)
    floor_us = statistics.median(fl)
    rows = [f"Launch floor (1 x 8 forward, 100 back-to-back launches from the host): {floor_us:.2f} us "
            "per launch.", "",
            "Per-kernel columns: HIP events around a run of back-to-back forwards, backwards (pass 1 + "
            "pass 2) or pass-1 launches (small shapes: host launch cost included). Graph columns: one "
            "captured step (forward, pass 1, pass 2) replayed back to back. Stream columns: the "
            "forward against a copy of the same tensor bytes, backward pass 1 against a two-input, "
            "one-output stream of the same tensor bytes (libdyt_streamref.so, measured alongside at "
            "that size): stream time / kernel time.", "",
            "| workload | M x N | x/params | fwd us | fwd GB/s | fwd % | bwd us | bwd GB/s | bwd % | "
            "step GB/s | step % | graph step us | graph GB/s | graph % | "
            "fwd / copy | pass 1 us | pass 1 / 2-in-1-out | plan |",
            "|---|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---|"]
    cold_rows = ["", "Cold cache: a 1 GiB buffer is read before each timed "
                 "launch; HIP events around the forward and around pass 1 + pass 2; median [p10, p90] over "
                 "30 repetitions. CPU oracle: the fp64 oracle as it is, per direction, on a sample of whole "
                 "rows (at most 2^20 elements), median of 3 runs on one pinned core of the host: "
                 + host_description() + ".", "",
                 "| workload | cold fwd us [p10, p90] | cold fwd GB/s | cold bwd us [p10, p90] | cold bwd GB/s | "
                 "oracle rows | oracle fwd GB/s | oracle bwd GB/s |",
                 "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for name in workloads.config_names():
        r = measure(dyt, torch, name, steps, warmup, graph=True, cold_iters=30)
        c = r["cold"]
        o = oracle_times(name)
        cold_rows.append(
            f"| {name} | {c['fwd']['p50_us']:.1f} [{c['fwd']['p10_us']:.1f}, {c['fwd']['p90_us']:.1f}] | "
            f"{c['fwd']['gbps']:.0f} | {c['bwd']['p50_us']:.1f} [{c['bwd']['p10_us']:.1f}, "
            f"{c['bwd']['p90_us']:.1f}] | {c['bwd']['gbps']:.0f} | {o['rows']} | {o['fwd_gbps']:.3f} | "
            f"{o['bwd_gbps']:.3f} |")
        log(cold_rows[-1])
        B = r["bytes"]
        step_us = r["fwd_us"] + r["bwd_us"]
        sgbps = (B["fwd"] + B["bwd"]) / (step_us * 1e-6) / 1e9
        tensor = r["M"] * r["N"] * (4 if r["x_dtype"] == "f32" else 2)
        sc = stream_ceilings(torch, max(tensor, 16))
        copy_us = 2 * sc["tensor_bytes"] / (sc["copy_GBps"] * 1e3)
        s21_us = 3 * sc["tensor_bytes"] / (sc["two_in_one_out_GBps"] * 1e3)
        def desc(pl, grid, fwd=False):
            if fwd and pl["flat"]:
                return f"flat, V={pl['vec']}, grid {pl['flat_grid']}"
            return (f"{'packed R=' + str(pl['rows_per_tile']) if pl['packed'] else 'rows nb=' + str(pl['col_blocks'])}"
                    f", V={pl['vec']} K={pl['slots']}, {pl['tiles']} tiles, grid {grid}")
        plan = (f"fwd: {desc(r['fwd_plan'], r['fwd_plan']['fwd_grid'], True)}; "
                f"bwd: {desc(r['plan'], r['plan']['bwd_grid'])}")
        rows.append(f"| {name} | {r['M']} x {r['N']} | {r['x_dtype']}/{r['param_dtype']} | "
                    f"{r['fwd_us']:.1f} | {r['fwd_gbps']:.0f} | {100 * r['fwd_frac']:.1f} | "
                    f"{r['bwd_us']:.1f} | {r['bwd_gbps']:.0f} | {100 * r['bwd_frac']:.1f} | "
                    f"{sgbps:.0f} | {100 * sgbps / HBM_PEAK_GBPS:.1f} | {r['graph_step_us']:.1f} | "
                    f"{r['graph_step_gbps']:.0f} | {100 * r['graph_step_gbps'] / HBM_PEAK_GBPS:.1f} | "
                    f"{copy_us / r['fwd_us']:.2f} | {r['pass1_us']:.1f} | "
                    f"{s21_us / r['pass1_us']:.2f} | {plan} |")
        log(rows[-1])
    with open(path, "w") as f:
        f.write("\n".join(rows + cold_rows) + "\n")


WIDTH_CASES = ([("bf16", n, 0) for n in (17, 255, 768, 1001, 1500, 1536, 2048, 2560, 3071, 3072, 4095, 4096,
                                        4104, 5120, 6144, 7168, 8192, 8200, 10240)]
               + [("f32", n, 0) for n in (1501, 2560, 4104, 5120, 9216, 13312)]
               + [("bf16", 4096, 1), ("bf16", 2560, 1), ("bf16", 1500, 1), ("bf16", 32, 1), ("f32", 100, 1)])


def parse_width_cases(spec: str | None) -> list:
    """'bf16:2560,f32:4104+1' -> [("bf16", 2560, 0), ("f32", 4104, 1)] (a '+1'
    suffix: bases one element off alignment); None -> every default case."""
    if not spec:
        return list(WIDTH_CASES)
    out = []
    for item in spec.split(","):
        xdt, n = item.strip().split(":")
        off = 1 if n.endswith("+1") else 0
        if xdt not in ("bf16", "f32"):
            raise ValueError(f"--width-cases: x dtype must be bf16 or f32, got {xdt!r}")
        out.append((xdt, int(n[:-2] if off else n), off))
    return out


def report_widths(dyt, torch, path: str, steps: int = 20, warmup: int = 5, rounds: int = 3,
                  cases=None) -> None:
    """Row widths that do not fill 4,096-element tiles, ragged rows and bases
    one element off 16-byte alignment, each at 2^27 elements (synthetic
    normal data, fp32 parameters): median over `rounds` of the mean forward
    and backward (pass 1 + pass 2) time of `steps` continuous calls (HIP
    events), with the plan each direction ran."""
    rows = ["Each case: 2^27 elements, x ~ N(0, 1), fp32 parameters; a settling run of "
            f"{SETTLE_S} s of forward + backward calls, then HIP events around "
            f"{steps} continuous calls after {warmup} warm-up calls, median of {rounds} rounds; "
            "backward = pass 1 + pass 2. Occupancy = share of the tile's vector slots that carry data.",
            "", "| x | N | M | base | fwd us | fwd GB/s | bwd us | bwd GB/s | fwd plan | bwd plan |",
            "|---|---:|---:|---|---:|---:|---:|---:|---|---|"]
    for xdt, N, off in (WIDTH_CASES if cases is None else cases):
        M = (1 << 27) // N
        dt = torch.bfloat16 if xdt == "bf16" else torch.float32
        gen = torch.Generator(device="cuda").manual_seed(N)

        def act():
            buf = torch.empty(M * N + 8, dtype=dt, device="cuda")
            v = buf[off:off + M * N].view(M, N)
            v.copy_(torch.randn(M, N, generator=gen, device="cuda"))
            return v
        x, dy, y, dx = act(), act(), act(), act()
        a = torch.tensor([0.5], device="cuda")
        g = torch.randn(N, generator=gen, device="cuda")
        b = torch.randn(N, generator=gen, device="cuda")
        da, dg, db = torch.empty(1, device="cuda"), torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
        ws = torch.empty(max(16, dyt.dyt_backward_workspace_size(M, N, xdt, "f32")), dtype=torch.uint8,
                         device="cuda")

        def fwd():
            dyt.dyt_forward(x, a, g, b, y=y)

        def bwd():
            dyt.dyt_backward(x, dy, a, g, dx=dx, dalpha=da, dgamma=dg, dbeta=db, workspace=ws)
        times = {}
        # settle the clocks on this case's own work before any timing
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            fwd()
            bwd()
            torch.cuda.synchronize()
        for key, fn in (("fwd", fwd), ("bwd", bwd)):
            med = []
            for _ in range(rounds):
                for _ in range(warmup):
                    fn()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    fn()
                e1.record()
                e1.synchronize()
                med.append(e0.elapsed_time(e1) * 1e3 / steps)
            times[key] = statistics.median(med)

        def desc(pl, fwd):
            cap = pl["block"] * pl["vec"] * pl["slots"]
            occ = pl["tile_elems"] / cap if pl["packed"] else N / (pl["col_blocks"] * cap)
            lay = f"packed R={pl['rows_per_tile']}" if pl["packed"] else f"rows nb={pl['col_blocks']}"
            # (every operand here is off by the same amount: the walk then starts aligned)
            if fwd and pl["flat"]:
                return f"flat walk, grid {pl['flat_grid']} (tiles: {lay}, K={pl['slots']}, occupancy {occ:.2f})"
            return f"{lay}, K={pl['slots']}, occupancy {occ:.2f}"
        sx = 2 if xdt == "bf16" else 4
        byt = M * N * sx
        rows.append(f"| {xdt} | {N} | {M} | {'+1 element' if off else 'aligned'} | {times['fwd']:.1f} | "
                    f"{2 * byt / times['fwd'] / 1e3:.0f} | {times['bwd']:.1f} | {3 * byt / times['bwd'] / 1e3:.0f} | "
                    f"{desc(dyt.dyt_get_forward_plan(M, N, xdt, 'f32'), True)} | {desc(dyt.dyt_get_plan(M, N, xdt, 'f32'), False)} |")
        log(rows[-1])
        del x, dy, y, dx, ws
    with open(path, "w") as f:
        f.write("\n".join(rows) + "\n")


TIMELINE_FLAGS = ["-DDYT_WG_TIMELINE=1"]


def timeline_library():
    """The library built with the workgroup timeline compiled in
    (bwd_dyt_forward_amd/libdyt_timeline.so; built here if missing or
    stale), loaded beside the default one with the same C signatures plus
    dyt_timeline_set."""
    import ctypes
    b = _build_module()
    path = os.path.join(ROOT, "bwd_dyt_forward_amd", "libdyt_timeline.so")
    if b.is_stale(path, TIMELINE_FLAGS):
        log("[bench] building the workgroup-timeline variant of the library")
        b.build(out=path, extra_flags=TIMELINE_FLAGS, with_stream_ref=False, cache=True)
    from bwd_dyt_forward_amd import _lib
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    for name, (res, argtypes) in _lib.SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = argtypes
    lib.dyt_timeline_set.restype = ctypes.c_int
    lib.dyt_timeline_set.argtypes = [ctypes.c_void_p]
    return lib


def _timeline_stats(st, tick_us: float) -> dict:
    """Summary of one launch's workgroup records st (G x 4 int64: entry,
    loop end, exit, ids), times in us from the earliest entry."""
    import numpy as np
    t = st[:, :3].astype(np.float64)
    t0 = t[:, 0].min()
    t = (t - t0) * tick_us
    xcc = (st[:, 3] >> 32) & 0xF
    ex = t[:, 2]
    per_xcd = {}
    for k in range(8):
        m = xcc == k
        if m.any():
            per_xcd[k] = (float(np.median(ex[m])), float(ex[m].max()), int(m.sum()),
                          float(np.median(t[m, 1] - t[m, 0])))
    # which XCD workgroup w ran on, as an offset k in XCD = (w + k) mod 8
    vals, counts = np.unique((xcc - np.arange(st.shape[0])) % 8, return_counts=True)
    return {
        "xcd_offset": int(vals[np.argmax(counts)]),
        "xcd_offset_all": bool(counts.max() == st.shape[0]),
        "span": float(ex.max()),
        "entry_spread": float(t[:, 0].max()),
        "exit_min": float(ex.min()), "exit_median": float(np.median(ex)), "exit_max": float(ex.max()),
        "end_phase": float(np.median(t[:, 2] - t[:, 1])),
        "tail": float(ex.max() - np.median(ex)),
        "per_xcd": per_xcd,
        "late": [(int(i), int(xcc[i]), float(ex[i])) for i in np.argsort(-ex)[:6]],
    }


def report_wg_timeline(torch, path: str, reps: int = 30,
                       names=(HEADLINE, SECONDARY), side_streams: int = 0, raw_dir: str | None = None) -> None:
    """Per-workgroup timeline of the forward and backward pass 1 in steady
    back-to-back steps (forward, pass 1, pass 2), from the timeline build of
    the library: when each workgroup starts, ends its streaming loop and
    exits, and on which XCD it ran. With side_streams, that many steps are
    first captured in HIP graphs on new streams and replayed (the state of
    a process that has used several streams). Writes a Markdown summary to
    path."""
    import numpy as np
    import workloads
    from bwd_dyt_forward_amd import _lib
    lib = timeline_library()
    tick_us = 0.01          # the real-time counter runs at 100 MHz
    rows = [f"# Workgroup timeline: forward and backward pass 1", "",
            f"Command: `python bench.py --wg-timeline {path} --timeline-workloads {','.join(names)}"
            + (f" --timeline-side-streams {side_streams}" if side_streams else "") + "` "
            f"(library built with {' '.join(TIMELINE_FLAGS)}; {reps} recorded steps after "
            f"{SETTLE_S} s of untimed steps; medians over the recorded steps). "
            f"Device: {torch.cuda.get_device_name(0)}.", "",
            "Times in us from the launch's earliest workgroup entry (real-time counter, "
            "100 MHz). span = last exit; tail = last exit - median exit; end phase = "
            "exit - end of the streaming loop (reduction and partial-row write in pass 1).", ""]
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    for name in names:
        inp = workloads.generate(name)
        xdt, pdt = tdt[inp.x_dtype], tdt[inp.p_dtype]
        dev = torch.device("cuda:0")
        x = torch.from_numpy(inp.x).to(dev).to(xdt)
        dy = torch.from_numpy(inp.dy).to(dev).to(xdt)
        a = torch.from_numpy(inp.alpha).to(dev).to(pdt)
        g = torch.from_numpy(inp.gamma).to(dev).to(pdt)
        b = torch.from_numpy(inp.beta).to(dev).to(pdt)
        M, N = inp.M, inp.N
        del inp
        y, dx = torch.empty_like(x), torch.empty_like(x)
        da = torch.empty(1, dtype=pdt, device=dev)
        dg = torch.empty(N, dtype=pdt, device=dev)
        db = torch.empty(N, dtype=pdt, device=dev)
        xc, pc = _lib._code(xdt), _lib._code(pdt)
        need = lib.dyt_backward_workspace_size(M, N, xc, pc)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        s = torch.cuda.current_stream()
        sp = s.cuda_stream
        pl = _lib.DytPlan()
        assert lib.dyt_get_plan(M, N, xc, pc, 1, ctypes_byref(pl)) == 0
        fpl = _lib.DytPlan()
        assert lib.dyt_get_forward_plan(M, N, xc, pc, 1, ctypes_byref(fpl)) == 0
        gf = fpl.flat_grid if fpl.flat else fpl.fwd_grid
        gb = pl.bwd_grid
        fst = torch.zeros((reps, gf, 4), dtype=torch.int64, device=dev)
        pst = torch.zeros((reps, gb, 4), dtype=torch.int64, device=dev)

        def step(r=None):
            lib.dyt_timeline_set(None if r is None else fst[r].data_ptr())
            assert lib.dyt_forward(x.data_ptr(), a.data_ptr(), g.data_ptr(), b.data_ptr(),
                                   y.data_ptr(), M, N, xc, pc, sp) == 0
            lib.dyt_timeline_set(None if r is None else pst[r].data_ptr())
            assert lib.dyt_backward_partials(x.data_ptr(), dy.data_ptr(), a.data_ptr(), g.data_ptr(),
                                             dx.data_ptr(), ws.data_ptr(), ws.numel(), M, N, xc, pc,
                                             sp) == 0
            lib.dyt_timeline_set(None)
            assert lib.dyt_backward_finish(ws.data_ptr(), ws.numel(), da.data_ptr(), dg.data_ptr(),
                                           db.data_ptr(), M, N, xc, pc, sp) == 0

        if side_streams:
            import bwd_dyt_forward_amd as dyt
            for _ in range(side_streams):
                graph_step_us(dyt, torch, x, dy, a, g, b, y, dx, ws, da, dg, db, M, N, xdt, reps=5)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            step()
        e1.record(s)
        e1.synchronize()
        plain_us = e0.elapsed_time(e1) * 1e3 / reps
        e0.record(s)
        for r in range(reps):
            step(r)
        e1.record(s)
        e1.synchronize()
        rec_us = e0.elapsed_time(e1) * 1e3 / reps
        fa, pa = fst.cpu().numpy(), pst.cpu().numpy()
        if raw_dir:
            os.makedirs(raw_dir, exist_ok=True)
            np.savez_compressed(os.path.join(raw_dir, f"{name}.npz"), forward=fa, pass1=pa)
        del x, dy, y, dx, ws, fst, pst
        torch.cuda.empty_cache()
        rows += [f"## {name} ({M} x {N})", "",
                 f"Step time (forward + pass 1 + pass 2): {plain_us:.1f} us without recording, "
                 f"{rec_us:.1f} us while recording.", ""]
        for kname, arr, grid in (("forward" + (" (flat walk)" if fpl.flat else ""), fa, gf),
                                 ("backward pass 1", pa, gb)):
            sts = [_timeline_stats(arr[r], tick_us) for r in range(reps)]
            med = lambda k: statistics.median(st[k] for st in sts)
            rows += [f"### {kname}: {grid} workgroups", "",
                     "| span | entry spread | first exit | median exit | last exit | tail | end phase |",
                     "|---:|---:|---:|---:|---:|---:|---:|",
                     f"| {med('span'):.2f} | {med('entry_spread'):.2f} | {med('exit_min'):.2f} | "
                     f"{med('exit_median'):.2f} | {med('exit_max'):.2f} | {med('tail'):.2f} | "
                     f"{med('end_phase'):.2f} |", "",
                     "| XCD | workgroups | median exit | last exit | median loop time |",
                     "|---:|---:|---:|---:|---:|"]
            for k in range(8):
                vals = [st["per_xcd"][k] for st in sts if k in st["per_xcd"]]
                if not vals:
                    continue
                rows.append(f"| {k} | {vals[0][2]} | {statistics.median(v[0] for v in vals):.2f} | "
                            f"{statistics.median(v[1] for v in vals):.2f} | "
                            f"{statistics.median(v[3] for v in vals):.2f} |")
            offs = {}
            for st in sts:
                key = st["xcd_offset"] if st["xcd_offset_all"] else "mixed"
                offs[key] = offs.get(key, 0) + 1
            rows += ["", "XCD of workgroup w as (w + k) mod 8, launches per k (mixed: no single k): " +
                     ", ".join(f"k = {k}: {n}" for k, n in sorted(offs.items(), key=lambda kv: str(kv[0])))]
            late = {}
            for st in sts:
                for i, k, _t in st["late"]:
                    late[(i, k)] = late.get((i, k), 0) + 1
            top = sorted(late.items(), key=lambda kv: -kv[1])[:8]
            rows += ["", "Workgroups most often among the six last to exit (index, XCD: times): " +
                     ", ".join(f"{i} (XCD {k}): {n}" for (i, k), n in top), ""]
        log(f"[bench] timeline {name}: step {plain_us:.1f} us plain, {rec_us:.1f} us recording")
    with open(path, "w") as f:
        f.write("\n".join(rows) + "\n")


# Library variants that --variants times against the default build: each a
# compile-time option of the sources, measured and not adopted (or, for
# default_constants, the tile table's own baseline).
VARIANTS = {
    # pass 1's last workgroup (by an arrival counter in the workspace) sums
    # the partial rows itself instead of a second launch
    "fused_finish": ["-DDYT_FUSED_FIN=1"],
    # plain loads and stores instead of nontemporal ones in both directions
    "no_nt_hints": ["-DDYT_FWD_NT=0", "-DDYT_BWD_NT=0"],
    # two tiles per pipeline buffer in pass 1 / one or four in the forward
    "bwd_two_units": ["-DDYT_BWD_U=2"],
    "fwd_one_unit": ["-DDYT_FWD_U=1"],
    "fwd_four_units": ["-DDYT_FWD_U=4"],
    # two tiles per buffer for the plain forward of 2-byte x as well
    "fwd_two_units_2b": ["-DDYT_FWD_U_2B=2"],
    # the flat forward on two or four workgroups per CU, or with eight
    # vectors per thread and step
    "flat_grid_512": ["-DDYT_FLAT_GRID=512"],
    "flat_grid_1024": ["-DDYT_FLAT_GRID=1024"],
    "flat_u8": ["-DDYT_FLAT_U=8"],
    # the flat forward for float32 rows however full their tiles are
    "flat_f32_all": ["-DDYT_FLAT_OCC_4B=1.01"],
    # float32 row segments keep their tiles at any size
    "flat_f32_big_off": ["-DDYT_FLAT_BIG_4B=4611686018427387904LL"],
    # pass 1's dx stores through a buffer descriptor with cache-policy bits:
    # sc0, sc1, sc1 + nontemporal
    "bwd_store_sc0": ["-DDYT_BWD_STORE_POL=1"],
    "bwd_store_sc1": ["-DDYT_BWD_STORE_POL=16"],
    "bwd_store_sc1_nt": ["-DDYT_BWD_STORE_POL=18"],
    # the default constants (one 256-thread workgroup per CU, largest tiles)
    # instead of the measured tile table
    "default_constants": ["-DDYT_TUNE_TABLE=0"],
    # the tiled forward everywhere (no flat walk)
    "no_flat_forward": ["-DDYT_FLAT_MAX_N=0"],
    # one-slot tiles (packed rows of one slot, row segments of one slot) on
    # 1,024 workgroups everywhere, and no flat walk
    "tiles_k1_g1024": ["-DDYT_TUNE_TABLE=0", "-DDYT_MIN_TILES=1048576", "-DDYT_WIDE_KCAP=1",
                       "-DDYT_FWD_GRID=1024", "-DDYT_FLAT_MAX_N=0"],
    # the forward's groups dealt round-robin to every workgroup instead of
    # the XCD-weighted deal
    "xcd_even_share_off": ["-DDYT_XCD_EVEN_SHARE_Q=0"],
    "xcd_even_share_56": ["-DDYT_XCD_EVEN_SHARE_Q=573"],
    # the 2-byte flat walk with the tiles' 53% share, or less
    "xcd_even_share_flat_53": ["-DDYT_XCD_EVEN_SHARE_FLAT_Q=543"],
    "xcd_even_share_flat_515": ["-DDYT_XCD_EVEN_SHARE_FLAT_Q=527"],
    "xcd_even_share_flat_52": ["-DDYT_XCD_EVEN_SHARE_FLAT_Q=532"],
    # backward pass 1 weighted too
    "xcd_even_share_bwd_51": ["-DDYT_XCD_EVEN_SHARE_BWD_Q=522"],
    "xcd_even_share_bwd_53": ["-DDYT_XCD_EVEN_SHARE_BWD_Q=543"],
    # nontemporal instead of write-back stores of the residual-fused pass 1's dh
    "bwd_res_nt": ["-DDYT_BWD_RES_NT=1"],
    # the persistent loops' earlier last load, which re-read the previous
    # group when a workgroup has an even number of groups
    "tail_prefetch": ["-DDYT_TAIL_PREFETCH=1"],
    # the tiled forward's first half of a grid of two workgroups per CU
    # (dispatched first) takes this share of the groups
    "round0_52": ["-DDYT_ROUND0_SHARE_Q=532"],
    "round0_535": ["-DDYT_ROUND0_SHARE_Q=548"],
    "round0_55": ["-DDYT_ROUND0_SHARE_Q=563"],
    # the forward's write-back stores: ordinary stores for float32 x too
    # (default: sc1, device-scope write-through buffer stores), or sc1 for
    # 2-byte x too (default: ordinary)
    "fwd_store_f32_plain": ["-DDYT_FWD_STORE_POL_F32=0"],
    "fwd_store_sc1_all": ["-DDYT_FWD_STORE_POL_2B=16"],
    # the float32 backward's longer small-|u| branch (tanh series through
    # u^13 and sech^2 = 1 - t^2 below |u| = 0.35)
    "bwd_f32_long_series": ["-DDYT_ACC_BWD_SERIES=1"],
}


def variant_library(name: str):
    """The library of a variant name: a VARIANTS entry (built from the
    current sources with its flags when stale), or lib:PATH, a prebuilt
    library of the same ABI from any sources (e.g. an earlier commit's)."""
    if name.startswith("lib:"):
        from bwd_dyt_forward_amd import _lib
        return _lib._load(name[4:], any_sources=True)
    flags = VARIANTS[name]
    b = _build_module()
    path = os.path.join(ROOT, "bwd_dyt_forward_amd", f"libdyt_variant_{name}.so")
    if b.is_stale(path, flags):
        log(f"[bench] building library variant {name} ({' '.join(flags)})")
        b.build(out=path, extra_flags=flags, with_stream_ref=False, cache=True)
    from bwd_dyt_forward_amd import _lib
    return _lib._load(path, flags)


def report_flat_crossover(dyt, torch, path: str, widths=(3072, 4096, 5120), rounds: int = 7) -> None:
    """Contiguous float32 forwards of row widths that fill their tiles
    (3,072 / 4,096 / 5,120), at sizes from 2^22 to 2^27 elements: their
    tiles (the flat_f32_big_off variant) against the flat walk (the
    flat_f32_all variant, which walks every such row flat), every output
    compared bit for bit, and which of the two the default plan takes; runs
    of back-to-back calls between two HIP events, the two libraries
    interleaved over rounds, medians. Writes Markdown."""
    import ctypes
    import statistics
    from bwd_dyt_forward_amd import _lib
    libs = {"tiles": variant_library("flat_f32_big_off"), "flat": variant_library("flat_f32_all")}
    s = torch.cuda.current_stream().cuda_stream
    sizes = (1 << 22, 1 << 24, 1 << 26, 80_000_000, 104_000_000, 1 << 27)
    rows = ["# Float32 forward: tiles against the flat walk by size", "",
            f"Command: `python bench.py --flat-crossover {path}"
            + ("" if tuple(widths) == (3072, 4096, 5120) else f" --flat-crossover-widths {','.join(map(str, widths))}")
            + f"`. Device: {torch.cuda.get_device_name(0)}. "
            f"Build id {dyt.lib.dyt_build_id().decode()}.", "",
            "us per call: a run of back-to-back forwards between two HIP events, the tiles (variant "
            f"flat_f32_big_off: {' '.join(VARIANTS['flat_f32_big_off'])}) and the flat walk (variant "
            f"flat_f32_all: {' '.join(VARIANTS['flat_f32_all'])}) interleaved over {rounds} rounds; "
            "medians. x ~ N(0, 1), fp32 parameters; y compared bit for bit. The default plan takes the "
            "flat walk for float32 row segments beyond 2^26 elements.", "",
            "| N | M | elements | tiles | tiles us | flat us | flat / tiles | default plan |",
            "|---:|---:|---:|---|---:|---:|---:|---|"]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for N in widths:
        for e in sizes:
            M = e // N
            x = torch.randn(M, N, device="cuda")
            a = torch.full((1,), 0.5, device="cuda")
            g = 1 + 0.1 * torch.randn(N, device="cuda")
            b = 0.1 * torch.randn(N, device="cuda")
            ys = {k: torch.empty_like(x) for k in libs}

            def call(k):
                return libs[k].dyt_forward(x.data_ptr(), a.data_ptr(), g.data_ptr(), b.data_ptr(),
                                           ys[k].data_ptr(), M, N, 0, 0, s)
            for k in libs:
                if call(k) != 0:
                    raise RuntimeError(f"forward failed on {M} x {N}")
            torch.cuda.synchronize()
            if not torch.equal(ys["tiles"], ys["flat"]):
                raise RuntimeError(f"the flat walk differs from the tiles on {M} x {N}")
            reps = max(5, int(20000 / (e / 2 ** 27 * 180 + 5)))
            t = {k: [] for k in libs}
            for rnd in range(rounds):
                for k in (list(libs) if rnd % 2 == 0 else list(libs)[::-1]):
                    for _ in range(3):
                        call(k)
                    e0.record()
                    for _ in range(reps):
                        call(k)
                    e1.record()
                    e1.synchronize()
                    t[k].append(e0.elapsed_time(e1) * 1e3 / reps)
            d, f = statistics.median(t["tiles"]), statistics.median(t["flat"])
            pt, pd = _lib.DytPlan(), _lib.DytPlan()
            libs["tiles"].dyt_get_forward_plan(M, N, 0, 0, 1, ctypes.byref(pt))
            dyt.lib.dyt_get_forward_plan(M, N, 0, 0, 1, ctypes.byref(pd))
            desc = f"{'packed' if pt.packed else 'rows'} nb={pt.col_blocks}, K={pt.slots}, grid {pt.fwd_grid}"
            if pt.flat:
                desc = "flat walk (tiles fill poorly)"
            rows.append(f"| {N:,} | {M:,} | {M * N:,} | {desc} | {d:.1f} | {f:.1f} | {f / d:.3f} | "
                        f"{'flat walk' if pd.flat else 'tiles'} |")
            log(f"[bench] flat crossover {M} x {N}: tiles {d:.1f} us, flat {f:.1f} us")
            del x, ys
            torch.cuda.empty_cache()
    with open(path, "w") as fh:
        fh.write("\n".join(rows) + "\n")


def report_variants(dyt, torch, path: str, names, rounds: int = 8) -> None:
    """Each named library variant against the default build on every
    workload, with its own forward and backward: the outputs compared bit
    for bit with the default build's, then back-to-back forwards, back-to-
    back backwards (both passes) and back-to-back steps (forward then
    backward), every library's run of each kind interleaved over rounds;
    medians. Writes Markdown."""
    import workloads
    from bwd_dyt_forward_amd import _lib
    libs = {"default": dyt.lib}
    for n in names:
        libs[n] = variant_library(n)
    rows = ["# Library variants against the default build", "",
            f"Command: `python bench.py --variants {','.join(names)} --variants-report {path}`. "
            f"Device: {torch.cuda.get_device_name(0)}.", "",
            "Variants (compile-time options of the same sources, or lib:PATH, a prebuilt library "
            "from other sources): " +
            "; ".join(f"`{n}`: " + (f"build id {libs[n].dyt_build_id().decode()}" if n.startswith("lib:")
                                   else ' '.join(VARIANTS[n])) for n in names) +
            f"; default: build id {dyt.lib.dyt_build_id().decode()}.", "",
            f"us per call: forward alone, backward (pass 1 + pass 2) alone and the step (forward then "
            f"backward), each a run of back-to-back calls between two HIP events; median of {rounds} "
            "rounds in which every library's run of each kind is interleaved. 'bits' compares y, dx, "
            "dgamma, dbeta and dalpha with the default build's.", "",
            "| workload | library | forward us | backward us | step us | step vs default | bits |",
            "|---|---|---:|---:|---:|---:|---|"]
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    dev = torch.device("cuda:0")
    s = torch.cuda.current_stream()
    sp = s.cuda_stream
    for name in workloads.config_names():
        inp = workloads.generate(name)
        xdt, pdt = tdt[inp.x_dtype], tdt[inp.p_dtype]
        x = torch.from_numpy(inp.x).to(dev).to(xdt)
        dy = torch.from_numpy(inp.dy).to(dev).to(xdt)
        a = torch.from_numpy(inp.alpha).to(dev).to(pdt)
        g = torch.from_numpy(inp.gamma).to(dev).to(pdt)
        b = torch.from_numpy(inp.beta).to(dev).to(pdt)
        M, N = inp.M, inp.N
        del inp
        xc, pc = _lib._code(xdt), _lib._code(pdt)
        bufs = {}
        for v, L in libs.items():
            need = L.dyt_backward_workspace_size(M, N, xc, pc)
            # zero-filled: a variant may keep counters in the workspace
            bufs[v] = (torch.zeros(max(need, 16), dtype=torch.uint8, device=dev), torch.empty_like(x),
                       torch.empty(1, dtype=pdt, device=dev), torch.empty(N, dtype=pdt, device=dev),
                       torch.empty(N, dtype=pdt, device=dev), torch.empty_like(x))

        def fwd(v):
            y = bufs[v][5]
            rc = libs[v].dyt_forward(x.data_ptr(), a.data_ptr(), g.data_ptr(), b.data_ptr(), y.data_ptr(),
                                     M, N, xc, pc, sp)
            if rc != 0:
                raise RuntimeError(f"variant {v}: dyt_forward returned {rc}")

        def bwd(v):
            ws, dx, da, dg, db, _y = bufs[v]
            rc = libs[v].dyt_backward(x.data_ptr(), dy.data_ptr(), a.data_ptr(), g.data_ptr(), dx.data_ptr(),
                                      da.data_ptr(), dg.data_ptr(), db.data_ptr(), ws.data_ptr(), ws.numel(),
                                      M, N, xc, pc, sp)
            if rc != 0:
                raise RuntimeError(f"variant {v}: dyt_backward returned {rc}")

        def step(v):
            fwd(v)
            bwd(v)

        same = {}
        for v in libs:
            for _ in range(2):
                step(v)
            torch.cuda.synchronize()
            same[v] = all(torch.equal(p.view(torch.uint8), q.view(torch.uint8))
                          for p, q in zip(bufs[v][1:], bufs["default"][1:]))
        reps = 10 if M * N >= (1 << 26) else 20
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            for v in libs:
                step(v)
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        kinds = {"fwd": fwd, "bwd": bwd, "step": step}
        us = {(v, k): [] for v in libs for k in kinds}
        order = list(libs)
        for r in range(rounds):
            for kname, fn in kinds.items():
                for j in range(len(order)):
                    v = order[(r + j) % len(order)]
                    e0.record(s)
                    for _ in range(reps):
                        fn(v)
                    e1.record(s)
                    e1.synchronize()
                    us[(v, kname)].append(e0.elapsed_time(e1) * 1e3 / reps)
        med = {key: statistics.median(val) for key, val in us.items()}
        for v in libs:
            rows.append(f"| {name} | {v} | {med[(v, 'fwd')]:.2f} | {med[(v, 'bwd')]:.2f} | "
                        f"{med[(v, 'step')]:.2f} | {med[(v, 'step')] / med[('default', 'step')]:.3f} | "
                        f"{'equal' if same[v] else 'differ'} |")
        log(f"[bench] variants {name}: " + ", ".join(f"{v} {med[(v, 'step')]:.2f}" for v in libs))
        del x, dy, bufs
        torch.cuda.empty_cache()
    rows += residual_variant_rows(torch, libs, rounds)
    with open(path, "w") as f:
        f.write("\n".join(rows) + "\n")


def residual_variant_rows(torch, libs, rounds: int) -> list:
    """The residual-fused layer (h = x + r, y = DyT(h); dh = dres + dx) of
    every library on the headline shape: forward alone, backward (both
    passes) alone and the step (forward then backward), interleaved as in
    report_variants; outputs compared bit for bit with the default build's."""
    import workloads
    from bwd_dyt_forward_amd import _lib
    inp = workloads.generate(HEADLINE)
    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    xdt, pdt = tdt[inp.x_dtype], tdt[inp.p_dtype]
    M, N = inp.M, inp.N
    x = torch.from_numpy(inp.x).to(dev).to(xdt)
    dy = torch.from_numpy(inp.dy).to(dev).to(xdt)
    a = torch.from_numpy(inp.alpha).to(dev).to(pdt)
    g = torch.from_numpy(inp.gamma).to(dev).to(pdt)
    b = torch.from_numpy(inp.beta).to(dev).to(pdt)
    del inp
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    r = torch.randn(M, N, generator=gen, device="cuda").to(xdt)
    dres = torch.randn(M, N, generator=gen, device="cuda").to(xdt)
    xc, pc = _lib._code(xdt), _lib._code(pdt)
    sp = torch.cuda.current_stream().cuda_stream
    bufs = {}
    for v, L in libs.items():
        need = L.dyt_backward_workspace_size(M, N, xc, pc)
        bufs[v] = {"ws": torch.zeros(max(need, 16), dtype=torch.uint8, device=dev),
                   "h": torch.empty_like(x), "y": torch.empty_like(x), "dh": torch.empty_like(x),
                   "da": torch.empty(1, dtype=pdt, device=dev), "dg": torch.empty(N, dtype=pdt, device=dev),
                   "db": torch.empty(N, dtype=pdt, device=dev)}

    def fwd(v):
        B = bufs[v]
        if libs[v].dyt_forward_residual(x.data_ptr(), r.data_ptr(), a.data_ptr(), g.data_ptr(), b.data_ptr(),
                                        B["h"].data_ptr(), B["y"].data_ptr(), M, N, xc, pc, sp) != 0:
            raise RuntimeError(f"variant {v}: dyt_forward_residual failed")

    def bwd(v):
        B = bufs[v]
        if libs[v].dyt_backward_residual(B["h"].data_ptr(), dy.data_ptr(), dres.data_ptr(), a.data_ptr(),
                                         g.data_ptr(), B["dh"].data_ptr(), B["da"].data_ptr(),
                                         B["dg"].data_ptr(), B["db"].data_ptr(), B["ws"].data_ptr(),
                                         B["ws"].numel(), M, N, xc, pc, sp) != 0:
            raise RuntimeError(f"variant {v}: dyt_backward_residual failed")

    def step(v):
        fwd(v)
        bwd(v)

    same = {}
    for v in libs:
        step(v)
        torch.cuda.synchronize()
        same[v] = all(torch.equal(bufs[v][k].view(torch.uint8), bufs["default"][k].view(torch.uint8))
                      for k in ("h", "y", "dh", "da", "dg", "db"))
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for v in libs:
            step(v)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    kinds = {"fwd": fwd, "bwd": bwd, "step": step}
    us = {(v, k): [] for v in libs for k in kinds}
    order = list(libs)
    for rr in range(rounds):
        for kname, fn in kinds.items():
            for j in range(len(order)):
                v = order[(rr + j) % len(order)]
                fn(v)
                e0.record()
                for _ in range(10):
                    fn(v)
                e1.record()
                e1.synchronize()
                us[(v, kname)].append(e0.elapsed_time(e1) * 1e3 / 10)
    med = {key: statistics.median(val) for key, val in us.items()}
    rows = ["", f"Residual-fused layer on {HEADLINE} (r and dres ~ N(0, 1), seed 1): forward, backward "
            "(both passes) and step (forward then backward) alone, us per call, medians as above.", "",
            "| library | forward us | backward us | step us | step vs default | bits |",
            "|---|---:|---:|---:|---:|---|"]
    for v in libs:
        rows.append(f"| {v} | {med[(v, 'fwd')]:.2f} | {med[(v, 'bwd')]:.2f} | {med[(v, 'step')]:.2f} | "
                    f"{med[(v, 'step')] / med[('default', 'step')]:.3f} | {'equal' if same[v] else 'differ'} |")
    del x, dy, r, dres, bufs
    torch.cuda.empty_cache()
    return rows


def report_placement(dyt, torch, path: str, name: str, variants=(), reps: int = 50) -> None:
    """The forward and backward pass 1 of one workload timed on tensors
    allocated at process start, after 8 s of steps on them, on the same
    shapes freed and allocated again, and again after an allocation churn
    (buffers of 1-600 MiB allocated, freed and returned to the driver), each
    after a 0.3 s settling run; HIP events around `reps` back-to-back
    launches, median of 3 runs; the default library and each named variant
    on the same tensors. Writes Markdown."""
    import workloads
    from bwd_dyt_forward_amd import _lib
    libs = {"default": dyt.lib}
    for v in variants:
        libs[v] = variant_library(v)
    cfg = workloads.CONFIGS[name]
    M, N = cfg.M, cfg.N
    xdt = {"f32": torch.float32, "bf16": torch.bfloat16}[cfg.x_dtype]
    pdt = {"f32": torch.float32, "bf16": torch.bfloat16}[cfg.p_dtype]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    a = torch.full((1,), 0.5, dtype=pdt, device="cuda")
    g = (1 + 0.02 * torch.randn(N, generator=gen, device="cuda")).to(pdt)
    b = torch.zeros(N, dtype=pdt, device="cuda")
    B = algorithmic_bytes(M, N, torch.empty((), dtype=xdt).element_size(), a.element_size())

    def alloc():
        x = torch.randn(M, N, generator=gen, device="cuda").to(xdt)
        dy = torch.randn(M, N, generator=gen, device="cuda").to(xdt)
        ws = torch.empty(max(dyt.dyt_backward_workspace_size(M, N, xdt, pdt), 16), dtype=torch.uint8,
                         device="cuda")
        return {"x": x, "dy": dy, "y": torch.empty_like(x), "dx": torch.empty_like(x), "ws": ws}

    def run(t, fn):
        out = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            fn(t)
            e0.record()
            for _ in range(reps):
                fn(t)
            e1.record()
            e1.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3 / reps)
        return statistics.median(out)

    xc, pc = _lib._code(xdt), _lib._code(pdt)
    s = torch.cuda.current_stream().cuda_stream

    def fwd_of(L):
        def f(t):
            if L.dyt_forward(t["x"].data_ptr(), a.data_ptr(), g.data_ptr(), b.data_ptr(), t["y"].data_ptr(),
                             M, N, xc, pc, s) != 0:
                raise RuntimeError("dyt_forward failed")
        return f

    def p1_of(L):
        def f(t):
            if L.dyt_backward_partials(t["x"].data_ptr(), t["dy"].data_ptr(), a.data_ptr(), g.data_ptr(),
                                       t["dx"].data_ptr(), t["ws"].data_ptr(), t["ws"].numel(), M, N, xc,
                                       pc, s) != 0:
                raise RuntimeError("dyt_backward_partials failed")
        return f

    fwd, p1 = fwd_of(dyt.lib), p1_of(dyt.lib)

    def settle(t, seconds=SETTLE_S):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                fwd(t)
                p1(t)
            torch.cuda.synchronize()

    rows = []

    def phase(label, t):
        settle(t)
        for v, L in libs.items():
            f, p = run(t, fwd_of(L)), run(t, p1_of(L))
            rows.append(f"| {label} | {v} | {f:.2f} | {B['fwd'] / (f * 1e-6) / 1e9:.0f} | {p:.2f} | "
                        f"{B['pass1'] / (p * 1e-6) / 1e9:.0f} |")
            log("[bench] placement: " + rows[-1])

    t = alloc()
    phase("tensors allocated at process start", t)
    settle(t, 8.0)
    phase("the same tensors after 8 s of forward + pass 1", t)
    t = None
    torch.cuda.empty_cache()
    t = alloc()
    phase("freed, returned to the driver and allocated again", t)
    for i in range(3):
        t = None
        torch.cuda.empty_cache()
        for mib in (1, 8, 40, 100, 300, 600, 300, 100, 8):
            z = [torch.empty(mib << 20, dtype=torch.uint8, device="cuda") for _ in range(3)]
            del z
            torch.cuda.empty_cache()
        t = alloc()
        phase(f"allocated again after an allocation churn ({i + 1})", t)
    # the other measurements of a workload in --all-configs, then eager again
    # on the same tensors
    da = torch.empty(1, dtype=pdt, device="cuda")
    dg = torch.empty(N, dtype=pdt, device="cuda")
    db = torch.empty(N, dtype=pdt, device="cuda")
    cold_times(dyt, torch, t["x"], t["dy"], a, g, b, t["y"], t["dx"], t["ws"], da, dg, db, M, N, xdt, 30, B)
    torch.cuda.empty_cache()
    phase("the same tensors after the cold-cache timing (1 GiB read before each launch)", t)
    graph_step_us(dyt, torch, t["x"], t["dy"], a, g, b, t["y"], t["dx"], t["ws"], da, dg, db, M, N, xdt)
    phase("the same tensors after a step captured in a HIP graph and replayed", t)
    stream_ceilings(torch, M * N * torch.empty((), dtype=xdt).element_size())
    phase("the same tensors after the reference streams", t)
    for _ in range(6):
        graph_step_us(dyt, torch, t["x"], t["dy"], a, g, b, t["y"], t["dx"], t["ws"], da, dg, db, M, N, xdt)
    phase("the same tensors after six more graph steps, each captured on a new stream", t)
    hdr = ["# Placement sensitivity: " + name, "",
           f"Command: `python bench.py --placement {path} --workload {name}"
           + (f" --placement-variants {','.join(variants)}" if variants else "") + "`. Device: "
           f"{torch.cuda.get_device_name(0)}.", "",
           "Each row: a 0.3 s settling run of forward + pass 1 calls on the tensors of that row, then "
           f"HIP events around {reps} back-to-back launches, median of 3 runs. The allocation churn "
           "allocates three buffers each of 1, 8, 40, 100, 300, 600, 300, 100 and 8 MiB in turn, "
           "freeing them and returning the memory to the driver after each size.", "",
           "| tensors | library | forward us | forward GB/s | pass 1 us | pass 1 GB/s |",
           "|---|---|---:|---:|---:|---:|"]
    with open(path, "w") as fh:
        fh.write("\n".join(hdr + rows) + "\n")


def graph_vs_eager(dyt, torch, name: str, steps: int = 50) -> dict:
    """The same step (forward, pass 1, pass 2) run eagerly and as a captured
    HIP graph: each phase a settling run of its own kind (0.3 s) followed at
    once by `steps` timed back-to-back steps, with a 50 ms idle gap between
    the two phases (so that a kernel trace of this run splits into them).
    Returns us per step for each."""
    import workloads
    inp = workloads.generate(name)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    xdt, pdt = tdt[inp.x_dtype], tdt[inp.p_dtype]
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp.x).to(dev).to(xdt)
    dy = torch.from_numpy(inp.dy).to(dev).to(xdt)
    a = torch.from_numpy(inp.alpha).to(dev).to(pdt)
    g = torch.from_numpy(inp.gamma).to(dev).to(pdt)
    b = torch.from_numpy(inp.beta).to(dev).to(pdt)
    M, N = inp.M, inp.N
    del inp
    y, dx = torch.empty_like(x), torch.empty_like(x)
    da = torch.empty(1, dtype=pdt, device=dev)
    dg = torch.empty(N, dtype=pdt, device=dev)
    db = torch.empty(N, dtype=pdt, device=dev)
    ws = torch.empty(max(16, dyt.dyt_backward_workspace_size(M, N, xdt, pdt)), dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream()

    def step():
        dyt.dyt_forward(x, a, g, b, y=y, stream=s)
        dyt.dyt_backward_partials(x, dy, a, g, dx, ws, stream=s)
        dyt.dyt_backward_finish(ws, M, N, xdt, da, dg, db, stream=s)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            for _ in range(20):
                step()
            s.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            step()
        for _ in range(5):
            graph.replay()
        s.synchronize()
        time.sleep(0.05)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        out = {}
        for phase in ("eager", "graph"):
            run = step if phase == "eager" else graph.replay
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < SETTLE_S:
                for _ in range(20):
                    run()
                s.synchronize()
            run()
            e0.record(s)
            for _ in range(steps):
                run()
            e1.record(s)
            e1.synchronize()
            out[phase] = e0.elapsed_time(e1) * 1e3 / steps
            time.sleep(0.05)
    return out


def graph_trace_summary(d: str, steps: int = 50) -> str:
    """From a rocprofv3 kernel trace of `bench.py --graph-vs-eager W`: the
    dispatches of the two timed phases (the last `steps` steps of the last
    two runs of DyT kernels separated by an idle gap; each run is a
    settling run followed by the timed steps), with each kernel family's
    mean duration and the mean gap from one kernel's end to the next one's
    start, per phase."""
    import csv
    import glob
    recs = []
    for fn in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                fam = _family(r["Kernel_Name"])
                if fam and fam != "calibration":
                    recs.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), fam))
    recs.sort()
    runs, cur = [], [recs[0]]
    for r in recs[1:]:
        if r[0] - cur[-1][1] > 10_000_000:      # an idle gap of more than 10 ms
            runs.append(cur)
            cur = []
        cur.append(r)
    runs.append(cur)
    lines = ["| phase | dispatches | " + " | ".join(f"{f} us" for f, _ in KERNEL_FAMILIES if f != "dyt_fwd_flat_kernel")
             + " | forward (flat) us | mean gap us | us per step |", "|---|---:|" + "---:|" * 6]
    for phase, run in zip(("eager", "graph"), runs[-2:]):
        run = run[-3 * steps:]                   # the timed steps: three kernels each
        dur = {}
        for st, en, fam in run:
            dur.setdefault(fam, []).append((en - st) / 1e3)
        gaps = [(run[i + 1][0] - run[i][1]) / 1e3 for i in range(len(run) - 1)]
        nsteps = max(1, len(dur.get("dyt_bwd_finish_kernel", [])))
        span = (run[-1][1] - run[0][0]) / 1e3
        m = lambda f: f"{statistics.mean(dur[f]):.2f}" if f in dur else "-"
        lines.append(f"| {phase} | {len(run)} | {m('dyt_fwd_kernel')} | {m('dyt_bwd_partial_kernel')} | "
                     f"{m('dyt_bwd_finish_kernel')} | {m('dyt_fwd_flat_kernel')} | "
                     f"{statistics.mean(gaps):.2f} | {span / nsteps:.2f} |")
    return "\n".join(lines)


def ctypes_byref(obj):
    import ctypes
    return ctypes.byref(obj)


# Kernel families, matched in the names the profiler records.
KERNEL_FAMILIES = (("dyt_fwd_flat_kernel", "dyt_fwd_flat_kernel<"), ("dyt_fwd_kernel", "dyt_fwd_kernel<"),
                   ("dyt_bwd_partial_kernel", "dyt_bwd_partial_kernel<"),
                   ("dyt_bwd_finish_kernel", "dyt_bwd_finish_kernel<"))
COUNTER_PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "sq": ["VALUBusy", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_WAVES", "SQ_INSTS_VMEM_RD",
           "SQ_INSTS_VMEM_WR", "SQ_INSTS_LDS"],
}


def _family(name: str):
    for fam, pat in KERNEL_FAMILIES:
        if pat in name:
            return fam
    return "calibration" if "neg_kernel" in name else None


def _read_counters(d: str) -> dict:
    """Mean value per dispatch of each counter, per kernel family, from the
    rocprofv3 CSV files under d (a counter spread over several rows of one
    dispatch is summed)."""
    import csv
    import glob
    per = {}
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                fam = _family(r["Kernel_Name"])
                if fam is None:
                    continue
                key = (fam, r["Counter_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    acc = {}
    for (fam, cn, _d), v in per.items():
        acc.setdefault(fam, {}).setdefault(cn, []).append(v)
    return {fam: {cn: sum(v) / len(v) for cn, v in cs.items()} for fam, cs in acc.items()}


def _read_trace_stats(d: str) -> dict:
    """Calls and mean duration (us) per kernel family from a rocprofv3
    --kernel-trace --stats run under d."""
    import csv
    import glob
    out = {}
    for fn in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                fam = _family(r["Name"])
                if fam is None or fam == "calibration":
                    continue
                calls, total = int(r["Calls"]), float(r["TotalDurationNs"])
                c0, t0 = out.get(fam, (0, 0.0))
                out[fam] = (c0 + calls, t0 + total)
    return {fam: {"calls": c, "mean_us": t / c / 1e3} for fam, (c, t) in out.items()}


def ingest_counters(root: str, calib_mib: int, md_path: str) -> None:
    """Reads the profiler output of `root/<workload>/{trace,fetch,write,sq}`
    (one directory per rocprofv3 pass over `bench.py --workload <workload>`;
    the counter passes with --copy-calibration-mib), scales the byte
    counters by what they read for the calibration copy of calib_mib MiB,
    and writes profiles/traffic_counters.json (per kernel and workload,
    tagged with the build id) and a Markdown summary."""
    import workloads
    h = kernel_source_hash()
    table = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            table = {k: v for k, v in json.load(f).items() if v.get("source_hash") == h}
    cal_bytes = calib_mib * (1 << 20)
    rows = ["# HBM bytes, VALU activity and kernel durations per workload", "",
            "Commands, per workload W (from the repository root; one profiler pass each):", "", "```",
            "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/pmc/W/trace -o W -- "
            "python3 bench.py --workload W --secondary none --no-residual --no-cpu-baseline --steps 20 --warmup 5"]
    for pname, cnts in COUNTER_PASSES.items():
        rows.append(f"rocprofv3 --pmc {' '.join(cnts)} --output-format csv -d gpurun_out/pmc/W/{pname} -o W -- "
                    f"python3 bench.py --workload W --secondary none --no-residual --no-cpu-baseline "
                    f"--steps 3 --warmup 1 --copy-calibration-mib {calib_mib}")
    rows += [f"python3 bench.py --ingest-counters gpurun_out/pmc --ingest-md {md_path}", "```", "",
             f"Byte counters are scaled by what they read for a plain elementwise copy of {calib_mib} MiB "
             "(torch.neg, reading and writing it once) in the same run. Counter values are means over "
             "every dispatch of the run; durations are the kernel trace's means. Algorithmic bytes: "
             "forward 2MN sx + (2N+1) sp, backward pass 1 3MN sx + (N+1) sp; pass 2 reads the "
             "workspace only. VALUBusy is the profiler's own derived metric; VALU and 2^x/1/x "
             "(transcendental) instructions are per element, counted per lane.", "",
             "| workload | kernel | trace us | GB/s | % of 8 TB/s | fetch MB | write MB | traffic / algorithmic "
             "| VALUBusy % | VALU inst / elem | transcendental / elem | LDS inst / elem |",
             "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for w in sorted(os.listdir(root)):
        wd = os.path.join(root, w)
        if w not in workloads.CONFIGS or not os.path.isdir(wd):
            continue
        cfg = workloads.CONFIGS[w]
        sx = 4 if cfg.x_dtype == "f32" else 2
        sp = 4 if cfg.p_dtype == "f32" else 2
        B = algorithmic_bytes(cfg.M, cfg.N, sx, sp)
        elems = cfg.M * cfg.N
        trace = _read_trace_stats(os.path.join(wd, "trace"))
        F = _read_counters(os.path.join(wd, "fetch"))
        W = _read_counters(os.path.join(wd, "write"))
        Q = _read_counters(os.path.join(wd, "sq"))
        ff = F.get("calibration", {}).get("FETCH_SIZE", 0) * 1024 / cal_bytes or None
        fw = W.get("calibration", {}).get("WRITE_SIZE", 0) * 1024 / cal_bytes or None
        for fam, _pat in KERNEL_FAMILIES:
            if fam not in trace and fam not in F:
                continue
            alg = {"dyt_fwd_flat_kernel": B["fwd"], "dyt_fwd_kernel": B["fwd"],
                   "dyt_bwd_partial_kernel": B["pass1"], "dyt_bwd_finish_kernel": None}[fam]
            ent = {"source_hash": h}
            fb = F.get(fam, {}).get("FETCH_SIZE")
            wb = W.get(fam, {}).get("WRITE_SIZE")
            if fb is not None and wb is not None and ff and fw:
                ent["fetch_bytes"] = round(fb * 1024 / ff)
                ent["write_bytes"] = round(wb * 1024 / fw)
                ent["bytes_per_launch"] = ent["fetch_bytes"] + ent["write_bytes"]
            q = Q.get(fam, {})
            if q:
                ent["valu_busy_pct"] = round(q.get("VALUBusy", float("nan")), 2)
                ent["valu_insts_per_elem"] = round(q.get("SQ_INSTS_VALU", 0) * 64 / elems, 3)
                ent["trans_insts_per_elem"] = round(q.get("SQ_INSTS_VALU_TRANS_F32", 0) * 64 / elems, 3)
                ent["lds_insts_per_elem"] = round(q.get("SQ_INSTS_LDS", 0) * 64 / elems, 3)
            if fam in trace:
                ent["trace_mean_us"] = round(trace[fam]["mean_us"], 2)
                ent["trace_calls"] = trace[fam]["calls"]
            if alg:
                ent["algorithmic_bytes"] = alg
            table[f"{fam}:{w}"] = ent
            t_us = ent.get("trace_mean_us")
            gbps = alg / (t_us * 1e-6) / 1e9 if (alg and t_us) else None
            f2 = lambda v, fmt: "-" if v is None else format(v, fmt)
            rows.append(
                f"| {w} | {fam} | {f2(t_us, '.2f')} | {f2(gbps, '.0f')} | "
                f"{f2(None if gbps is None else 100 * gbps / HBM_PEAK_GBPS, '.1f')} | "
                f"{f2(ent.get('fetch_bytes', None) and ent['fetch_bytes'] / 1e6, '.1f')} | "
                f"{f2(ent.get('write_bytes', None) and ent['write_bytes'] / 1e6, '.1f')} | "
                f"{f2(alg and ent.get('bytes_per_launch') and ent['bytes_per_launch'] / alg, '.3f')} | "
                f"{f2(ent.get('valu_busy_pct'), '.1f')} | {f2(ent.get('valu_insts_per_elem'), '.2f')} | "
                f"{f2(ent.get('trans_insts_per_elem'), '.2f')} | {f2(ent.get('lds_insts_per_elem'), '.3f')} |")
    rows += ["", f"Build id of the measured library: `{h}`; bench.py reports these figures only while "
             "the sources still have this id."]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    with open(md_path, "w") as f:
        f.write("\n".join(rows) + "\n")


def load_traffic(kernel: str) -> dict | None:
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--secondary", default=SECONDARY, help="second workload reported alongside ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    ap.add_argument("--no-residual", action="store_true",
                    help="skip the residual-fused vs unfused comparison")
    ap.add_argument("--all-configs", metavar="FILE", default=None,
                    help="also time every workload shape and write a Markdown table to FILE")
    ap.add_argument("--widths", metavar="FILE", default=None,
                    help="also time awkward row widths and unaligned bases and write a Markdown table to FILE")
    ap.add_argument("--width-cases", default=None,
                    help="with --widths: only these cases, e.g. 'bf16:2560,f32:4104,bf16:4096+1'")
    ap.add_argument("--wg-timeline", metavar="FILE", default=None,
                    help="only record the per-workgroup timeline of the forward and backward pass 1 "
                         "(timeline build of the library) and write a Markdown summary to FILE")
    ap.add_argument("--timeline-workloads", default=f"{HEADLINE},{SECONDARY}",
                    help="with --wg-timeline: comma-separated workload names")
    ap.add_argument("--timeline-raw", metavar="DIR", default=None,
                    help="with --wg-timeline: also save every recorded launch's per-workgroup words "
                         "(entry, loop end, exit, XCC_ID << 32 | HW_ID) as DIR/<workload>.npz")
    ap.add_argument("--timeline-side-streams", type=int, default=0,
                    help="with --wg-timeline: first capture and replay this many steps in HIP graphs "
                         "on new streams")
    ap.add_argument("--ingest-counters", metavar="DIR", default=None,
                    help="only read the profiler output under DIR/<workload>/{trace,fetch,write,sq} and "
                         "write profiles/traffic_counters.json and the Markdown summary --ingest-md")
    ap.add_argument("--ingest-md", default=os.path.join("profiles", "dyt_kernels_counters.md"))
    ap.add_argument("--graph-vs-eager", metavar="WORKLOAD", default=None,
                    help="only time WORKLOAD's step eagerly and as a replayed HIP graph (for a kernel trace)")
    ap.add_argument("--graph-trace", metavar="DIR", default=None,
                    help="only summarise a kernel trace of --graph-vs-eager found under DIR (no GPU)")
    ap.add_argument("--variants", default=None,
                    help="only time these library variants (comma-separated names of VARIANTS, "
                         "or lib:PATH for a prebuilt library from other sources) against the "
                         "default build on every workload")
    ap.add_argument("--variants-report", metavar="FILE", default="variants.md")
    ap.add_argument("--flat-crossover", metavar="FILE", default=None,
                    help="only time float32 forwards of full-tile widths by size, their tiles "
                         "(variant flat_f32_big_off) against the flat walk (variant flat_f32_all), "
                         "and write Markdown")
    ap.add_argument("--flat-crossover-widths", default="3072,4096,5120",
                    help="row widths of --flat-crossover (comma-separated)")
    ap.add_argument("--placement", metavar="FILE", default=None,
                    help="only time the --workload's forward and pass 1 on tensors allocated at "
                         "process start, after sustained steps and after reallocation (Markdown to FILE)")
    ap.add_argument("--placement-variants", default="",
                    help="with --placement: also time these library variants (comma-separated)")
    args = ap.parse_args()

    if args.graph_trace:
        print(graph_trace_summary(args.graph_trace))
        return 0
    if args.ingest_counters:
        ingest_counters(args.ingest_counters, args.copy_calibration_mib or 1024, args.ingest_md)
        log(f"[bench] counters written to {TRAFFIC_FILE} and {args.ingest_md}")
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the DyT layer runs on one MI355X here; the row-sharded design is described, not run.",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import __graft_entry__ as ge
    ge._ensure_built()
    import bwd_dyt_forward_amd as dyt

    if args.graph_vs_eager:
        r = graph_vs_eager(dyt, torch, args.graph_vs_eager)
        log(f"[bench] {args.graph_vs_eager}: eager {r['eager']:.2f} us per step, graph {r['graph']:.2f} us per step")
        return 0
    if args.flat_crossover:
        report_flat_crossover(dyt, torch, args.flat_crossover,
                              tuple(int(v) for v in args.flat_crossover_widths.split(",")))
        log(f"[bench] flat crossover written to {args.flat_crossover}")
        return 0
    if args.variants:
        report_variants(dyt, torch, args.variants_report, args.variants.split(","))
        log(f"[bench] variant report written to {args.variants_report}")
        return 0
    if args.placement:
        report_placement(dyt, torch, args.placement, args.workload,
                         [v for v in args.placement_variants.split(",") if v])
        log(f"[bench] placement report written to {args.placement}")
        return 0
    if args.wg_timeline:
        report_wg_timeline(torch, args.wg_timeline, names=args.timeline_workloads.split(","),
                           side_streams=args.timeline_side_streams, raw_dir=args.timeline_raw)
        log(f"[bench] workgroup timeline written to {args.wg_timeline}")
        return 0

    main_res = measure(dyt, torch, args.workload, args.steps, args.warmup)
    log(f"[bench] {json.dumps(main_res)}")
    sec = None
    if args.secondary and args.secondary != "none" and args.secondary != args.workload:
        sec = measure(dyt, torch, args.secondary, args.steps, args.warmup)
        log(f"[bench] {json.dumps(sec)}")
    resid = None
    if not args.no_residual:
        resid = measure_residual(dyt, torch, args.workload)
        rsc = residual_stream_ceilings(torch, main_res["M"] * main_res["N"] *
                                       (2 if main_res["x_dtype"] in ("bf16", "f16") else 4))
        resid["stream_ceiling"] = rsc
        resid["fwd"]["frac_of_2in2out"] = round(resid["fwd"]["fused_GBps"] / rsc["2in2out_GBps"], 4)
        resid["bwd"]["frac_of_3in1out"] = round(resid["bwd"]["fused_GBps"] / rsc["3in1out_GBps"], 4)
        log(f"[bench] residual: {json.dumps(resid)}")
    if args.copy_calibration_mib:
        copy_calibration(torch, args.copy_calibration_mib)
    if args.all_configs:
        report_all(dyt, torch, args.all_configs)
    if args.widths:
        report_widths(dyt, torch, args.widths, cases=parse_width_cases(args.width_cases))

    tensor_bytes = main_res["M"] * main_res["N"] * (2 if main_res["x_dtype"] in ("bf16", "f16") else 4)
    ceiling = copy_ceiling(torch, tensor_bytes)
    log(f"[bench] device copy ceiling: {ceiling:.1f} GB/s")
    streams = stream_ceilings(torch, tensor_bytes)
    streams["fwd_frac_of_copy"] = round(main_res["fwd_gbps"] / streams["copy_GBps"], 4)
    streams["pass1_frac_of_2in1out"] = round(main_res["pass1_gbps"] / streams["two_in_one_out_GBps"], 4)
    log(f"[bench] stream ceilings: {json.dumps(streams)}")
    kernel = "dyt_bwd_partial_kernel"
    traffic = load_traffic(kernel + ":" + args.workload)
    rl_bytes = main_res["bytes"]["pass1"]
    achieved = main_res["pass1_gbps"]
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": None if traffic is None else traffic.get("bytes_per_launch"),
        "kernel": kernel, "algorithmic_bytes_per_launch": rl_bytes,
        "mean_launch_us": round(main_res["pass1_us"], 2),
    }
    # The same kernel's mean duration in the committed kernel trace of this
    # workload (profiles/dyt_kernels_counters.md), while the sources are
    # those it measured: the events' run of back-to-back launches includes
    # the dispatch gaps between launches, the trace does not.
    if traffic is not None and traffic.get("trace_mean_us"):
        t_us = traffic["trace_mean_us"]
        roofline["trace_mean_us"] = t_us
        roofline["trace_achieved"] = round(rl_bytes / (t_us * 1e-6) / 1e9, 1)
        roofline["trace_frac"] = round(rl_bytes / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        roofline["counters"] = "profiles/dyt_kernels_counters.md"
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, args.cpu_seconds)
    out = {
        "metric": "DyT fwd+bwd effective HBM GB/s and % of MI355X peak, per (M,N,dtype)",
        "value": round(main_res["gbps_step"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "warmup_steps_run": main_res["warmup_steps_run"],
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": main_res["M"], "N": main_res["N"],
                   "x_dtype": main_res["x_dtype"], "param_dtype": main_res["param_dtype"],
                   "parallelism": "single GPU"},
        "frac_of_peak": round(main_res["gbps_step"] / HBM_PEAK_GBPS, 4),
        "copy_ceiling_GBps": round(ceiling, 1),
        "stream_ceiling": streams,
        "fwd": {"GBps": round(main_res["fwd_gbps"], 1), "frac": round(main_res["fwd_frac"], 4),
                "us": round(main_res["fwd_us"], 2)},
        "bwd": {"GBps": round(main_res["bwd_gbps"], 1), "frac": round(main_res["bwd_frac"], 4),
                "us": round(main_res["bwd_us"], 2),
                "pass2_us": round(main_res["pass2_us"], 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if sec:
        out["secondary"] = {
            "workload": sec["workload"], "GBps": round(sec["gbps_step"], 1),
            "frac": round(sec["gbps_step"] / HBM_PEAK_GBPS, 4),
            "fwd": {"GBps": round(sec["fwd_gbps"], 1), "frac": round(sec["fwd_frac"], 4),
                    "us": round(sec["fwd_us"], 2)},
            "bwd": {"GBps": round(sec["bwd_gbps"], 1), "frac": round(sec["bwd_frac"], 4),
                    "us": round(sec["bwd_us"], 2)},
        }
    if resid:
        out["residual"] = resid
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
