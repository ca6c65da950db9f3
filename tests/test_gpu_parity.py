"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every workload shape is compared element by element: the small ones at
their full size, the two 134M-element ones at reduced row counts (several
tiles plus a ragged tail) and at full size on sampled y/dx elements with
the parameter gradients against the oracle's full sums. Tolerances are the
ones stated in oracle/compare.py (float32 rel 1e-6 on y and dx; bfloat16
within 1 ulp of the rounded oracle; gradients rel 1e-5 at the terms' RSS)."""
import pytest
import torch

import workloads
from gpu_util import (assert_reports, every_element_reports, full_reports, log, run_both,
                      sampled_reports, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dyt():
    import __graft_entry__ as ge
    ge._ensure_built()
    import bwd_dyt_forward_amd as m
    return m


FULL_SIZE = ["c1_1024x64_f32", "c2_65537x16_bf16", "c3_100003x17_f32_inf",
             "c3_100003x100_f32_inf", "c3_100003x255_f32_inf"]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_parity_full_size(dyt, name):
    log(f"[parity full] {name}")
    inp = workloads.generate(name)
    outs = run_both(dyt, upload(inp))
    assert_reports(name, full_reports(inp, *outs))


REDUCED = [("c4_32768x4096_bf16", 37), ("c4_32768x4096_bf16", 1),
           ("c5_4194304x32_bf16_outliers", 20001), ("c5_4194304x32_bf16_outliers", 129),
           ("c2_65537x16_bf16", 1000), ("c3_100003x255_f32_inf", 77), ("c1_1024x64_f32", 3)]


@pytest.mark.parametrize("name,M", REDUCED)
def test_parity_reduced_rows(dyt, name, M):
    log(f"[parity reduced] {name} M={M}")
    inp = workloads.generate(name, M=M)
    outs = run_both(dyt, upload(inp))
    assert_reports(f"{name}[M={M}]", full_reports(inp, *outs))


@pytest.mark.parametrize("name", ["c4_32768x4096_bf16", "c5_4194304x32_bf16_outliers"])
def test_parity_full_size_sampled(dyt, name):
    log(f"[parity full sampled] {name}")
    inp = workloads.generate(name)
    d = upload(inp)
    outs = run_both(dyt, d)
    assert_reports(name, sampled_reports(inp, *outs))
    del d, outs
    torch.cuda.empty_cache()


SWEEP = [
    # (M, N, x dtype, param dtype, alpha): packed, wide, multi-block and ragged-row paths
    (257, 1, "f32", "f32", 0.7), (513, 3, "bf16", "f32", 1.1), (97, 250, "bf16", "f32", 0.5),
    (41, 300, "bf16", "f32", 0.5), (33, 1000, "f32", "f32", 0.9), (9, 2049, "bf16", "f32", 0.5),
    (7, 4100, "bf16", "f32", 0.5), (5, 8192, "bf16", "f32", 0.5), (3, 20000, "f32", "f32", 0.3),
    (301, 64, "f32", "bf16", 0.5), (300, 4096, "bf16", "bf16", 0.5), (1031, 17, "bf16", "bf16", 2.0),
    (4099, 8, "f32", "f32", 3.0), (1, 7, "f32", "f32", 0.5),
    # float16 activations and/or parameters
    (65537, 16, "f16", "f32", 0.8), (37, 4096, "f16", "f32", 0.5), (1031, 300, "f16", "f16", 1.5),
    (513, 17, "f32", "f16", 0.9), (257, 64, "bf16", "f16", 0.7), (9, 4100, "f16", "bf16", 0.5),
    # negative alpha (a learnable scale may change sign)
    (1003, 255, "f32", "f32", -0.7), (300, 4096, "bf16", "f32", -1.3),
]


@pytest.mark.parametrize("M,N,xdt,pdt,alpha", SWEEP)
def test_parity_shape_sweep(dyt, M, N, xdt, pdt, alpha):
    log(f"[parity sweep] M={M} N={N} x={xdt} p={pdt} alpha={alpha} plan={dyt.dyt_get_plan(M, N, xdt, pdt)}")
    inp = workloads.custom(M, N, xdt, pdt, alpha=alpha, x_sigma=2.0, seed=M + N)
    outs = run_both(dyt, upload(inp))
    assert_reports(inp.name, full_reports(inp, *outs))


@pytest.mark.parametrize("name", ["c4_32768x4096_bf16", "c5_4194304x32_bf16_outliers"])
def test_parity_full_size_every_element(dyt, name, capsys):
    """All 134,217,728 elements of y and dx at the full size and launch plan
    the benchmark times, each against the oracle, plus the gradients. The
    reports go to the terminal even when pytest captures output."""
    import time
    t0 = time.perf_counter()
    log(f"[parity full every element] {name}")
    inp = workloads.generate(name)
    d = upload(inp)
    outs = run_both(dyt, d)
    del d
    log(f"  inputs and GPU run {time.perf_counter() - t0:.1f} s")
    reps = every_element_reports(inp, *outs)
    log(f"  oracle comparison done at {time.perf_counter() - t0:.1f} s")
    assert reps[0].n == inp.M * inp.N and reps[1].n == inp.M * inp.N
    del outs
    torch.cuda.empty_cache()
    with capsys.disabled():
        for rep in reps:
            print(f"\n  [every element] {name}: {rep}", flush=True)
    assert_reports(name, reps)
