"""Seeded synthetic inputs for the fused Dynamic Tanh (DyT) layer.

This module only draws and quantises input data. It holds none of the
layer's arithmetic, so both the fp64 CPU oracle (through the tests) and the
HIP library (through the tests and the benchmark) consume exactly the same
stored bits without sharing any code of the method.

The workloads are the five shapes on which the layer is measured and
checked (the Liger-Kernel pull request "fix(dyt): use a 1D grid and tile
small-width rows" motivates each of them in its Summary and Testing Done
sections: more than 65,535 rows, narrow and ragged widths, infinite alpha,
bfloat16 input with float32 parameters):

  c1  1024 x 64,          fp32 x/params, x,dy ~ N(0,1), alpha 0.5
  c2  65,537 x 16,        bf16 x, fp32 params, alpha 0.8
  c3  100,003 x {17,100,255}, fp32, x,dy ~ N(0, sigma=2), alpha = +inf
  c4  32,768 x 4,096,     bf16 x, fp32 params, alpha 0.5, beta = 0
  c5  4,194,304 x 32,     bf16 x, fp32 params, 1% outliers at +-50, alpha 1

Recipe (fixed so results are reproducible): ``numpy.random.default_rng(seed)``
(PCG64), drawn in this order: x, dy, gamma, beta, then x's outlier mask and
signs, then dy's. Normal draws are float64, scaled, cast to float32 with
round-to-nearest-even (RNE), and for bfloat16 tensors rounded again to
bfloat16 with RNE on the float32 bit pattern. ``N(mu, s)`` means standard
deviation ``s``. Large tensors are drawn in row chunks; sequential chunked
draws from one generator give the same stream as a single draw.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["CONFIGS", "Inputs", "generate", "bf16_round_bits", "config_names"]

_CHUNK_ELEMS = 1 << 24


@dataclass(frozen=True)
class Config:
    name: str
    M: int
    N: int
    x_dtype: str          # "f32" | "bf16" | "f16"
    p_dtype: str          # "f32" | "bf16" | "f16"
    x_sigma: float        # standard deviation of x and dy
    alpha: float
    gamma: tuple          # ("normal", mean, sd) | ("uniform", lo, hi)
    beta: tuple           # ("normal", mean, sd) | ("zero",)
    outlier_p: float = 0.0
    outlier_mag: float = 0.0
    note: str = ""


CONFIGS: dict[str, Config] = {
    c.name: c
    for c in [
        Config("c1_1024x64_f32", 1024, 64, "f32", "f32", 1.0, 0.5,
               ("normal", 1.0, 0.1), ("normal", 0.0, 0.1),
               note="small fp32 case"),
        Config("c2_65537x16_bf16", 65537, 16, "bf16", "f32", 1.0, 0.8,
               ("normal", 1.0, 0.1), ("normal", 0.0, 0.1),
               note="more rows than a 65,535-block grid dimension"),
        Config("c3_100003x17_f32_inf", 100003, 17, "f32", "f32", 2.0, float("inf"),
               ("uniform", 0.5, 1.5), ("normal", 0.0, 0.1),
               note="ragged width, infinite alpha"),
        Config("c3_100003x100_f32_inf", 100003, 100, "f32", "f32", 2.0, float("inf"),
               ("uniform", 0.5, 1.5), ("normal", 0.0, 0.1),
               note="ragged width, infinite alpha"),
        Config("c3_100003x255_f32_inf", 100003, 255, "f32", "f32", 2.0, float("inf"),
               ("uniform", 0.5, 1.5), ("normal", 0.0, 0.1),
               note="ragged width, infinite alpha"),
        Config("c4_32768x4096_bf16", 32768, 4096, "bf16", "f32", 1.0, 0.5,
               ("normal", 1.0, 0.02), ("zero",),
               note="transformer block: 8 x 4096 tokens, hidden 4096"),
        Config("c5_4194304x32_bf16_outliers", 4194304, 32, "bf16", "f32", 1.0, 1.0,
               ("normal", 1.0, 0.1), ("normal", 0.0, 0.1),
               outlier_p=0.01, outlier_mag=50.0,
               note="small-network bulk, 1% outliers at +-50 in x and dy"),
    ]
}


def config_names() -> list[str]:
    return list(CONFIGS)


@dataclass
class Inputs:
    """One workload instance. Arrays hold the exact stored values.

    ``x`` and ``dy`` are float32 arrays of shape (M, N) whose values are
    exactly representable in ``x_dtype``; ``alpha`` (shape (1,)), ``gamma``
    and ``beta`` (shape (N,)) are float32 arrays exactly representable in
    ``p_dtype``.
    """
    name: str
    x: np.ndarray
    dy: np.ndarray
    alpha: np.ndarray
    gamma: np.ndarray
    beta: np.ndarray
    x_dtype: str
    p_dtype: str
    meta: dict = field(default_factory=dict)

    @property
    def M(self) -> int:
        return self.x.shape[0]

    @property
    def N(self) -> int:
        return self.x.shape[1]


def bf16_round_bits(f32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Only used to quantise finite synthetic inputs; NaN inputs are not
    expected here and are quieted.
    """
    b = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    nan = np.isnan(f32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    r = ((b + bias) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def _bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _quantise(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return a32
    if dtype == "bf16":
        return _bits_to_f32(bf16_round_bits(a32))
    if dtype == "f16":
        return np.asarray(a32, dtype=np.float32).astype(np.float16).astype(np.float32)
    raise ValueError(f"unsupported dtype {dtype!r}")


def _normal_matrix(rng: np.random.Generator, M: int, N: int, sigma: float,
                   dtype: str) -> np.ndarray:
    out = np.empty((M, N), dtype=np.float32)
    flat = out.reshape(-1)
    total = M * N
    pos = 0
    while pos < total:
        n = min(_CHUNK_ELEMS, total - pos)
        z = rng.standard_normal(n) * sigma
        flat[pos:pos + n] = _quantise(z.astype(np.float32), dtype)
        pos += n
    return out


def _apply_outliers(rng: np.random.Generator, a: np.ndarray, p: float,
                    mag: float) -> int:
    """Replace each element with probability p by +-mag (fair-coin sign)."""
    flat = a.reshape(-1)
    total = flat.size
    pos = 0
    count = 0
    while pos < total:
        n = min(_CHUNK_ELEMS, total - pos)
        hit = rng.random(n) < p
        neg = rng.random(n) < 0.5
        vals = np.where(neg, -mag, mag).astype(np.float32)
        seg = flat[pos:pos + n]
        seg[hit] = vals[hit]
        count += int(hit.sum())
        pos += n
    return count


def _param(rng: np.random.Generator, spec: tuple, N: int, dtype: str) -> np.ndarray:
    kind = spec[0]
    if kind == "normal":
        v = spec[1] + spec[2] * rng.standard_normal(N)
    elif kind == "uniform":
        v = rng.uniform(spec[1], spec[2], N)
    elif kind == "zero":
        v = np.zeros(N)
    else:
        raise ValueError(kind)
    return _quantise(v.astype(np.float32), dtype)


def generate(name: str, seed: int = 0, M: int | None = None) -> Inputs:
    """Draw the inputs of workload ``name``.

    ``M`` overrides the row count (same distributions, fewer or more rows);
    used for reduced-size parity cases.
    """
    cfg = CONFIGS[name]
    M = cfg.M if M is None else int(M)
    N = cfg.N
    rng = np.random.default_rng(seed)
    x = _normal_matrix(rng, M, N, cfg.x_sigma, cfg.x_dtype)
    dy = _normal_matrix(rng, M, N, cfg.x_sigma, cfg.x_dtype)
    gamma = _param(rng, cfg.gamma, N, cfg.p_dtype)
    beta = _param(rng, cfg.beta, N, cfg.p_dtype)
    meta = {"seed": seed, "config": name}
    if cfg.outlier_p > 0:
        meta["x_outliers"] = _apply_outliers(rng, x, cfg.outlier_p, cfg.outlier_mag)
        meta["dy_outliers"] = _apply_outliers(rng, dy, cfg.outlier_p, cfg.outlier_mag)
    alpha = _quantise(np.array([cfg.alpha], dtype=np.float32), cfg.p_dtype)
    meta["x_exact_zeros"] = int(np.count_nonzero(x == 0))
    return Inputs(name, x, dy, alpha, gamma, beta, cfg.x_dtype, cfg.p_dtype, meta)


def from_arrays(x, dy, alpha, gamma, beta, x_dtype: str, p_dtype: str,
                name: str = "custom") -> Inputs:
    """Wrap hand-made arrays (already representable in their dtypes)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    for arr, dt in ((x, x_dtype), (dy, x_dtype)):
        if dt != "f32" and not np.array_equal(_quantise(arr, dt), arr, equal_nan=True):
            raise ValueError(f"values not representable in {dt}")
    return Inputs(name, x, dy,
                  np.ascontiguousarray(alpha, dtype=np.float32).reshape(1),
                  np.ascontiguousarray(gamma, dtype=np.float32),
                  np.ascontiguousarray(beta, dtype=np.float32),
                  x_dtype, p_dtype, {})


def custom(M: int, N: int, x_dtype: str = "f32", p_dtype: str = "f32", alpha: float = 0.5,
           x_sigma: float = 1.0, seed: int = 0) -> Inputs:
    """Extra shapes for parity sweeps: x, dy ~ N(0, x_sigma), gamma ~ N(1, 0.1),
    beta ~ N(0, 0.1), same draw order and quantisation as the named workloads."""
    rng = np.random.default_rng(seed)
    x = _normal_matrix(rng, M, N, x_sigma, x_dtype)
    dy = _normal_matrix(rng, M, N, x_sigma, x_dtype)
    gamma = _param(rng, ("normal", 1.0, 0.1), N, p_dtype)
    beta = _param(rng, ("normal", 0.0, 0.1), N, p_dtype)
    a = _quantise(np.array([alpha], dtype=np.float32), p_dtype)
    return Inputs(f"custom_{M}x{N}_{x_dtype}_{p_dtype}", x, dy, a, gamma, beta, x_dtype, p_dtype,
                  {"seed": seed})


def residual_pair(M: int, N: int, x_dtype: str, seed: int, sigma: float = 1.0):
    """Extra tensors of the residual-fused layer: r (the branch output added
    to the residual stream x) and dres (the gradient reaching h through the
    residual stream), both ~ N(0, sigma) in x_dtype, drawn in that order from
    their own generator (seed + 1000003) so the layer's own inputs stay those
    of the workload."""
    rng = np.random.default_rng(seed + 1000003)
    r = _normal_matrix(rng, M, N, sigma, x_dtype)
    dres = _normal_matrix(rng, M, N, sigma, x_dtype)
    return r, dres
