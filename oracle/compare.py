"""Rounding helpers and tolerance checks against the fp64 DyT oracle.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this module.

Tolerances (stated per output; every check also demands that NaN appears
at exactly the positions where the oracle has NaN, and that infinities
match exactly):

* y, float32:  |y_gpu - y*| <= 1e-6 * S_y, with S_y = |gamma t| + |beta|.
  Measuring against the condition scale keeps a near-cancelling
  gamma*t + beta from demanding more than the inputs determine.
* y, bfloat16: |y_gpu - rne_bf16(y*)| <= 1 ulp_bf16(max(|y*|, S_y)).
* dx, float32: |dx_gpu - dx*| <= 1e-6 * |dx*| + floor, where floor covers
  intermediate float32 underflow of sech^2 (|alpha x| > ~43.7, where
  float32 keeps fewer than 24 bits): floor = 2^-149 * (1 + 4 |dy gamma alpha|).
* dx, bfloat16: |dx_gpu - rne_bf16(dx*)| <= 1 ulp_bf16(|dx*|).
* float16 outputs follow the bfloat16 rules with float16 rounding and ulps
  (11 significant bits, subnormal spacing 2^-24, overflow to +-inf).
* dh of the residual backward (dres + dx, one rounding): the y rules with
  the scale S_dh = |dres| + |dx*|, plus the float32 dx underflow floor.
* h of the residual forward (x + r rounded once): exact, bit for bit.
* dgamma, dbeta, dalpha (float32 accumulation):
  |g_gpu - g*| <= 1e-5 * max(|g*|, RSS_g) + 2^-149, RSS_g the root sum of
  squares of the summed terms (random-sign sums are compared at the scale
  the inputs fix, not at an accidental near-zero total). bfloat16 params:
  |g_gpu - rne_bf16(g*)| <= 1 ulp_bf16(|g*|) + 1e-5 * RSS_g.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rne_bf16", "ulp_bf16", "rne_f16", "ulp_f16", "rne", "ulp", "Report",
    "check_y", "check_dx", "check_grad", "check_dh", "check_exact",
]

_BF16_OVERFLOW = 2.0 ** 128
_F32_TINY = 2.0 ** -149


def rne_bf16(v) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits, float32's
    exponent range, subnormal spacing 2^-133), round-to-nearest-even, in one
    step (no intermediate float32 rounding). NaN and +-inf pass through;
    values that round past the largest finite bfloat16 become +-inf."""
    v0 = np.asarray(v, dtype=np.float64)
    v = np.atleast_1d(v0)
    out = v.copy()
    fin = np.isfinite(v)
    a = np.abs(v[fin])
    _, e = np.frexp(a)                       # a = m * 2^e, m in [0.5, 1)
    sp = np.maximum(e - 8, -133)             # exponent of the bf16 spacing
    q = np.rint(np.ldexp(a, -sp))            # exact scaling; rint is RNE
    r = np.ldexp(q, sp)
    r[r >= _BF16_OVERFLOW] = np.inf
    out[fin] = np.copysign(r, v[fin])
    return out.reshape(v0.shape)


def ulp_bf16(v) -> np.ndarray:
    """Spacing of bfloat16 values at magnitude |v|: 2^(floor(log2|v|) - 7)
    for normal values, 2^-133 below 2^-126 (subnormals and zero)."""
    a0 = np.abs(np.asarray(v, dtype=np.float64))
    a = np.atleast_1d(a0)
    _, e = np.frexp(a)
    e = np.where(a == 0, -126, e)            # frexp(0) reports exponent 0
    u = np.ldexp(np.ones_like(a), np.maximum(e - 8, -133))
    u[~np.isfinite(a)] = np.inf
    return u.reshape(a0.shape)


def rne_f16(v) -> np.ndarray:
    """Round float64 values to IEEE binary16 (11 significant bits, subnormal
    spacing 2^-24, largest finite 65504), round-to-nearest-even, in one step
    on the scaled integer grid (no intermediate float32 rounding); values that
    round past 65504 become +-inf."""
    v0 = np.asarray(v, dtype=np.float64)
    v = np.atleast_1d(v0)
    out = v.copy()
    fin = np.isfinite(v)
    a = np.abs(v[fin])
    _, e = np.frexp(a)
    sp = np.maximum(e - 11, -24)
    q = np.rint(np.ldexp(a, -sp))
    r = np.ldexp(q, sp)
    r[r >= 65520.0] = np.inf          # 65504 + half its spacing rounds to even = inf
    out[fin] = np.copysign(r, v[fin])
    return out.reshape(v0.shape)


def ulp_f16(v) -> np.ndarray:
    """Spacing of float16 values at magnitude |v| (2^-24 below 2^-14)."""
    a0 = np.abs(np.asarray(v, dtype=np.float64))
    a = np.atleast_1d(a0)
    _, e = np.frexp(a)
    e = np.where(a == 0, -14, e)
    u = np.ldexp(np.ones_like(a), np.maximum(e - 11, -24))
    u[~np.isfinite(a)] = np.inf
    return u.reshape(a0.shape)


def rne(v, dtype: str) -> np.ndarray:
    """Round float64 values to the given storage dtype (RNE), as float64."""
    if dtype == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return rne_bf16(v)
    if dtype == "f16":
        return rne_f16(v)
    raise ValueError(dtype)


def ulp(v, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return ulp_bf16(v)
    if dtype == "f16":
        return ulp_f16(v)
    raise ValueError(dtype)


@dataclass
class Report:
    name: str
    n: int
    n_fail: int = 0
    nan_mismatch: int = 0
    inf_mismatch: int = 0
    worst_ratio: float = 0.0          # max err / bound over finite elements
    first_fail: list = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return self.n_fail == 0 and self.nan_mismatch == 0 and self.inf_mismatch == 0

    def __str__(self) -> str:
        return (f"{self.name}: n={self.n} fail={self.n_fail} nan_mismatch={self.nan_mismatch} "
                f"inf_mismatch={self.inf_mismatch} worst_err/bound={self.worst_ratio:.3g} "
                f"first={self.first_fail[:5]}")


def _finish(name, got, ref_cmp, bound) -> Report:
    got = np.asarray(got, dtype=np.float64).reshape(-1)
    ref_cmp = np.asarray(ref_cmp, dtype=np.float64).reshape(-1)
    bound = np.asarray(bound, dtype=np.float64)
    bound = bound.reshape(-1) if bound.size == got.size else np.broadcast_to(bound, got.shape)
    rep = Report(name, got.size)
    gnan, rnan = np.isnan(got), np.isnan(ref_cmp)
    rep.nan_mismatch = int(np.count_nonzero(gnan != rnan))
    ginf, rinf = np.isinf(got), np.isinf(ref_cmp)
    both_inf = ginf & rinf
    rep.inf_mismatch = int(np.count_nonzero(ginf != rinf)) + \
        int(np.count_nonzero(got[both_inf] != ref_cmp[both_inf]))
    fin = np.isfinite(got) & np.isfinite(ref_cmp)
    err = np.abs(got[fin] - ref_cmp[fin])
    b = bound[fin]
    bad = err > b
    rep.n_fail = int(np.count_nonzero(bad))
    if err.size:
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(b > 0, err / b, np.where(err > 0, np.inf, 0.0))
        rep.worst_ratio = float(np.max(ratio))
    if rep.n_fail or rep.nan_mismatch:
        idx = np.flatnonzero(fin)[np.flatnonzero(bad)][:5].tolist()
        idx += np.flatnonzero(gnan != rnan)[:5].tolist()
        rep.first_fail = idx
    return rep


def check_y(got, y_ref, scale, dtype: str, name: str = "y") -> Report:
    y_ref = np.asarray(y_ref, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    if dtype == "f32":
        return _finish(name, got, y_ref, 1e-6 * scale)
    if dtype in ("bf16", "f16"):
        return _finish(name, got, rne(y_ref, dtype),
                       ulp(np.maximum(np.abs(y_ref), scale), dtype))
    raise ValueError(dtype)


def check_dx(got, dx_ref, dtype: str, dy_gamma_alpha=None, name: str = "dx") -> Report:
    """dx is a pure product, so its scale is |dx*| itself.

    ``dy_gamma_alpha`` (|dy * gamma * alpha| per element) sizes the float32
    underflow floor; omit it when |alpha x| stays below ~43."""
    dx_ref = np.asarray(dx_ref, dtype=np.float64)
    if dtype == "f32":
        k = 0.0 if dy_gamma_alpha is None else 4.0 * np.abs(np.asarray(dy_gamma_alpha, np.float64))
        return _finish(name, got, dx_ref, 1e-6 * np.abs(dx_ref) + _F32_TINY * (1.0 + k))
    if dtype in ("bf16", "f16"):
        return _finish(name, got, rne(dx_ref, dtype), ulp(dx_ref, dtype))
    raise ValueError(dtype)


def check_grad(got, g_ref, rss, dtype: str, name: str = "grad") -> Report:
    g_ref = np.atleast_1d(np.asarray(g_ref, dtype=np.float64))
    rss = np.atleast_1d(np.asarray(rss, dtype=np.float64))
    got = np.atleast_1d(np.asarray(got, dtype=np.float64))
    if dtype == "f32":
        return _finish(name, got, g_ref, 1e-5 * np.maximum(np.abs(g_ref), rss) + _F32_TINY)
    if dtype in ("bf16", "f16"):
        return _finish(name, got, rne(g_ref, dtype), ulp(g_ref, dtype) + 1e-5 * rss)
    raise ValueError(dtype)


def check_dh(got, dh_ref, scale, dtype: str, dy_gamma_alpha=None, name: str = "dh") -> Report:
    """dh = dres + dx: a sum that can cancel, judged at its condition scale
    |dres| + |dx*| (like y), with dx's float32 underflow floor."""
    dh_ref = np.asarray(dh_ref, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    if dtype == "f32":
        k = 0.0 if dy_gamma_alpha is None else 4.0 * np.abs(np.asarray(dy_gamma_alpha, np.float64))
        return _finish(name, got, dh_ref, 1e-6 * scale + _F32_TINY * (1.0 + k))
    if dtype in ("bf16", "f16"):
        return _finish(name, got, rne(dh_ref, dtype), ulp(np.maximum(np.abs(dh_ref), scale), dtype))
    raise ValueError(dtype)


def check_exact(got, ref, name: str = "h") -> Report:
    """Bit-for-bit equality of values (NaN where NaN; -0 and +0 compared as
    values; zero tolerance)."""
    return _finish(name, got, ref, 0.0)
