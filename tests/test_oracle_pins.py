"""Pins of the fp64 DyT oracle against facts that do not come from the oracle.

Each pin rests on something independent of the oracle's own code:
closed forms (alpha = 0, the identity tanh(ln k) = (k^2-1)/(k^2+1)), a
library routine (math.tanh), complex-step and central-difference
derivatives of the oracle's *forward* (which pin the hand-written
backward), exact integer sums done with Python integers, the IEEE table in
tests/golden/alpha_inf_ieee.txt (the "Padding" bullet of the Liger-Kernel
pull request "fix(dyt): use a 1D grid and tile small-width rows"), and
brute-force per-element loops. ``test_pins_catch_planted_mistakes`` plants
plausible mistakes into the oracle on the CPU and checks that at least one
pin fails for each.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.dyt_oracle as O
from oracle import compare as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- pins
# Each pin raises AssertionError on failure. They call the oracle only via
# the module object so that test_pins_catch_planted_mistakes can patch it.

def pin_alpha_zero_gives_beta(o):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 7))
    g, b = rng.standard_normal(7), rng.standard_normal(7)
    r = o.forward(x, [0.0], g, b)
    assert np.array_equal(r.y, np.broadcast_to(b, (5, 7))), "alpha=0 must give y=beta exactly"
    bw = o.backward(x, rng.standard_normal((5, 7)), [0.0], g)
    assert np.array_equal(bw.dx, np.zeros((5, 7))), "alpha=0 must give dx=0"
    assert np.array_equal(bw.dgamma, np.zeros(7)), "alpha=0 must give dgamma=0"


def pin_unit_affine_is_library_tanh(o):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 6)) * 3
    a = 0.7
    r = o.forward(x, [a], np.ones(6), np.zeros(6))
    want = np.array([[math.tanh(a * v) for v in row] for row in x])
    assert np.allclose(r.y, want, rtol=4e-16, atol=0), "gamma=1, beta=0 must give tanh(alpha x)"


def pin_rational_points(o):
    """u = ln k gives tanh u = (k^2-1)/(k^2+1), sech^2 u = 4k^2/(k^2+1)^2."""
    ks = np.arange(2, 12)
    a = 0.5
    x = (2.0 * np.log(ks.astype(np.float64)))[None, :]      # alpha*x = ln k
    g = np.linspace(0.5, 1.5, ks.size)
    b = np.linspace(-0.3, 0.3, ks.size)
    dy = np.linspace(-2.0, 2.0, ks.size)[None, :]
    t = np.array([float(Fraction(k * k - 1, k * k + 1)) for k in ks])
    s = np.array([float(Fraction(4 * k * k, (k * k + 1) ** 2)) for k in ks])
    r = o.forward(x, [a], g, b)
    assert np.allclose(r.y[0], g * t + b, rtol=1e-14, atol=1e-15), "y at rational points"
    bw = o.backward(x, dy, [a], g)
    assert np.allclose(bw.dx[0], dy[0] * g * a * s, rtol=1e-13, atol=0), "dx at rational points"
    assert np.allclose(bw.dgamma, dy[0] * t, rtol=1e-14, atol=1e-16), "dgamma at rational points"
    assert np.allclose(bw.dbeta, dy[0], rtol=0, atol=0), "dbeta at rational points"
    dal = float(np.sum(dy[0] * g * x[0] * s))
    assert math.isclose(bw.dalpha, dal, rel_tol=1e-13), "dalpha at rational points"


def _complex_step_grads(o, x, dy, a, g, b, h=1e-30):
    """d(sum dy*y)/dp for every input p, by complex-step on o.forward_core."""
    def L(xx, aa, gg, bb):
        return np.sum(dy * o.forward_core(xx, aa, gg, bb))
    M, N = x.shape
    xc = x.astype(np.complex128)
    gx = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            xp = xc.copy()
            xp[i, j] += 1j * h
            gx[i, j] = L(xp, a, g, b).imag / h
    ga = L(xc, a + 1j * h, g, b).imag / h
    gg = np.empty(N)
    gb = np.empty(N)
    for j in range(N):
        e = np.zeros(N, dtype=np.complex128)
        e[j] = 1j * h
        gg[j] = L(xc, a, g + e, b).imag / h
        gb[j] = L(xc, a, g, b + e).imag / h
    return gx, ga, gg, gb


def pin_complex_step(o):
    rng = np.random.default_rng(3)
    M, N = 3, 5                                   # M != N catches axis mix-ups
    x = rng.standard_normal((M, N)) * 1.5
    dy = rng.standard_normal((M, N))
    g = 1 + 0.2 * rng.standard_normal(N)
    b = 0.1 * rng.standard_normal(N)
    a = 0.8
    gx, ga, gg, gb = _complex_step_grads(o, x, dy, a, g, b)
    bw = o.backward(x, dy, [a], g)
    assert np.allclose(bw.dx, gx, rtol=1e-12, atol=1e-15), "dx vs complex step"
    assert math.isclose(bw.dalpha, ga, rel_tol=1e-12), "dalpha vs complex step"
    assert np.allclose(bw.dgamma, gg, rtol=1e-12, atol=1e-15), "dgamma vs complex step"
    assert np.allclose(bw.dbeta, gb, rtol=1e-12, atol=1e-15), "dbeta vs complex step"


def pin_central_differences(o):
    rng = np.random.default_rng(4)
    M, N = 4, 3
    x = rng.standard_normal((M, N))
    dy = rng.standard_normal((M, N))
    g = 1 + 0.3 * rng.standard_normal(N)
    b = 0.2 * rng.standard_normal(N)
    a = 1.3

    def L(xx, aa, gg, bb):
        return float(np.sum(dy * o.forward(xx, [aa], gg, bb).y))
    bw = o.backward(x, dy, [a], g)
    for i in range(M):
        for j in range(N):
            h = 1e-6 * max(1.0, abs(x[i, j]))
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            fd = (L(xp, a, g, b) - L(xm, a, g, b)) / (2 * h)
            assert math.isclose(bw.dx[i, j], fd, rel_tol=1e-6, abs_tol=1e-9), "dx vs FD"
    h = 1e-6
    fd = (L(x, a + h, g, b) - L(x, a - h, g, b)) / (2 * h)
    assert math.isclose(bw.dalpha, fd, rel_tol=1e-6, abs_tol=1e-9), "dalpha vs FD"
    for j in range(N):
        e = np.zeros(N)
        e[j] = 1e-6
        fdg = (L(x, a, g + e, b) - L(x, a, g - e, b)) / 2e-6
        fdb = (L(x, a, g, b + e) - L(x, a, g, b - e)) / 2e-6
        assert math.isclose(bw.dgamma[j], fdg, rel_tol=1e-6, abs_tol=1e-9), "dgamma vs FD"
        assert math.isclose(bw.dbeta[j], fdb, rel_tol=1e-6, abs_tol=1e-9), "dbeta vs FD"


def pin_integer_sums_alpha_inf(o):
    """alpha=+inf, nonzero x, integer dy: dgamma_j = sum dy*sign(x),
    dbeta_j = sum dy, dalpha = 0, dx all NaN (exact, Python integers)."""
    rng = np.random.default_rng(5)
    M, N = 37, 6
    x = rng.standard_normal((M, N))
    x[x == 0] = 1.0
    dy = rng.integers(-3, 4, size=(M, N)).astype(np.float64)
    g = rng.uniform(0.5, 1.5, N)
    bw = o.backward(x, dy, [np.inf], g)
    for j in range(N):
        sg = sum(int(dy[i, j]) * (1 if x[i, j] > 0 else -1) for i in range(M))
        sb = sum(int(dy[i, j]) for i in range(M))
        assert bw.dgamma[j] == sg, "dgamma with alpha=inf"
        assert bw.dbeta[j] == sb, "dbeta with alpha=inf"
    assert bw.dalpha == 0.0, "dalpha with alpha=inf must be exactly 0"
    assert np.isnan(bw.dx).all(), "dx with alpha=inf must be NaN everywhere"


def pin_integer_sums_alpha_zero(o):
    """alpha=0, integer x, dy, gamma: dalpha = sum dy*gamma*x exactly."""
    rng = np.random.default_rng(6)
    M, N = 29, 5
    x = rng.integers(-2, 3, size=(M, N)).astype(np.float64)
    dy = rng.integers(-3, 4, size=(M, N)).astype(np.float64)
    g = rng.integers(1, 3, size=N).astype(np.float64)
    bw = o.backward(x, dy, [0.0], g)
    want = sum(int(dy[i, j]) * int(g[j]) * int(x[i, j]) for i in range(M) for j in range(N))
    assert bw.dalpha == want, "dalpha with alpha=0"
    for j in range(N):
        assert bw.dbeta[j] == sum(int(dy[i, j]) for i in range(M)), "dbeta column sum"


def _load_ieee_table():
    rows = []
    with open(os.path.join(GOLDEN, "alpha_inf_ieee.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([float(v) for v in line.split()])
    return np.array(rows)


def pin_ieee_alpha_inf_table(o):
    tab = _load_ieee_table()
    for row in tab:
        xv, dyv, gv, bv, y_w, dx_w, tg_w, tb_w, ta_w = row
        x = np.array([[xv]])
        dy = np.array([[dyv]])
        r = o.forward(x, [np.inf], [gv], [bv])
        bw = o.backward(x, dy, [np.inf], [gv])
        for got, want, what in ((r.y[0, 0], y_w, "y"), (bw.dx[0, 0], dx_w, "dx"),
                                (bw.dgamma[0], tg_w, "dgamma"), (bw.dbeta[0], tb_w, "dbeta"),
                                (bw.dalpha, ta_w, "dalpha")):
            if math.isnan(want):
                assert math.isnan(got), f"{what} must be NaN for x={xv}"
            else:
                assert got == want, f"{what}={got} != {want} for x={xv}"


def pin_large_u_sech2_not_cancelled(o):
    """|alpha x| = 30: 1 - tanh^2 rounds to 0 in fp64, but sech^2 = 4e^-60(1+e^-60)^-2."""
    for u in (20.0, 30.0, -30.0, 200.0):
        bw = o.backward(np.array([[u]]), np.array([[1.0]]), [1.0], [1.0])
        want = 4.0 * math.exp(-2 * abs(u)) / (1 + math.exp(-2 * abs(u))) ** 2
        assert math.isclose(bw.dx[0, 0], want, rel_tol=1e-13), f"sech^2 at u={u}"


def pin_odd_symmetry(o):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 4)) * 2
    g = rng.standard_normal(4)
    r1 = o.forward(x, [0.9], g, np.zeros(4))
    r2 = o.forward(-x, [0.9], g, np.zeros(4))
    assert np.array_equal(r2.y, -r1.y), "y - beta must be odd in x"


def pin_bruteforce_sums(o):
    """Sums and scales against per-element scalar loops with math.fsum."""
    rng = np.random.default_rng(8)
    M, N = 7, 3
    x = rng.standard_normal((M, N)) * 2
    dy = rng.standard_normal((M, N))
    g = 1 + 0.1 * rng.standard_normal(N)
    b = 0.1 * rng.standard_normal(N)
    a = 0.6
    bw = o.backward(x, dy, [a], g)
    r = o.forward(x, [a], g, b)
    for j in range(N):
        tg = [dy[i, j] * math.tanh(a * x[i, j]) for i in range(M)]
        assert math.isclose(bw.dgamma[j], math.fsum(tg), rel_tol=1e-14), "dgamma column sum"
        assert math.isclose(bw.rss_dgamma[j], math.sqrt(math.fsum(v * v for v in tg)), rel_tol=1e-14)
        assert math.isclose(bw.dbeta[j], math.fsum(dy[:, j]), rel_tol=1e-14), "dbeta column sum"
        for i in range(M):
            t = math.tanh(a * x[i, j])
            assert math.isclose(r.scale[i, j], abs(g[j] * t) + abs(b[j]), rel_tol=1e-15)
    ta = [dy[i, j] * g[j] * x[i, j] / math.cosh(a * x[i, j]) ** 2 for i in range(M) for j in range(N)]
    assert math.isclose(bw.dalpha, math.fsum(ta), rel_tol=1e-13), "dalpha full sum"
    assert math.isclose(bw.rss_dalpha, math.sqrt(math.fsum(v * v for v in ta)), rel_tol=1e-13)


def pin_empty(o):
    bw = o.backward(np.zeros((0, 5)), np.zeros((0, 5)), [0.5], np.ones(5))
    assert bw.dgamma.shape == (5,) and not bw.dgamma.any() and not bw.dbeta.any()
    assert bw.dalpha == 0.0
    bw = o.backward(np.zeros((3, 0)), np.zeros((3, 0)), [0.5], np.ones(0))
    assert bw.dalpha == 0.0 and bw.dgamma.shape == (0,)


def pin_sampled_matches_full(o):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((9, 6))
    dy = rng.standard_normal((9, 6))
    g, b = 1 + rng.standard_normal(6) * 0.1, rng.standard_normal(6) * 0.1
    r = o.forward(x, [0.5], g, b)
    bw = o.backward(x, dy, [0.5], g)
    rows, cols = np.divmod(np.arange(54), 6)
    ys, ss = o.forward_at(x[rows, cols], cols, [0.5], g, b)
    assert np.array_equal(ys, r.y.reshape(-1)) and np.array_equal(ss, r.scale.reshape(-1))
    dxs = o.backward_dx_at(x[rows, cols], dy[rows, cols], cols, [0.5], g)
    assert np.array_equal(dxs, bw.dx.reshape(-1))


# --- residual add fused in front of the layer (h = x + r rounded once, y from h)

def pin_residual_zero_branch(o):
    """r = +-0: h is x itself and y is the plain layer's y."""
    rng = np.random.default_rng(21)
    x = C.rne_bf16(rng.standard_normal((5, 7)))
    g, b = 1 + rng.standard_normal(7) * 0.1, rng.standard_normal(7) * 0.1
    for z in (0.0, -0.0):
        h, f = o.forward_residual(x, np.full((5, 7), z), [0.7], g, b, "bf16")
        assert np.array_equal(h, x)
        assert np.array_equal(f.y, o.forward(x, [0.7], g, b).y)


def pin_residual_integer_sums(o):
    """Integer-valued x and r: h is the exact integer sum (Python ints)."""
    rng = np.random.default_rng(22)
    xi = rng.integers(-100, 101, (6, 5))
    ri = rng.integers(-100, 101, (6, 5))
    for dt in ("f32", "bf16", "f16"):
        h, _ = o.forward_residual(xi.astype(np.float64), ri.astype(np.float64), [0.5], np.ones(5),
                                  np.zeros(5), dt)
        want = [[int(a) + int(c) for a, c in zip(ra, rr)] for ra, rr in zip(xi.tolist(), ri.tolist())]
        # |sum| <= 200 has at most 8 significant bits: exact in every dtype
        assert h.tolist() == want


def pin_residual_rounding_ties(o):
    """Hand-worked round-to-nearest-even of x + r, and y taken from h as stored."""
    cases = [  # (dtype, x, r, h)
        ("bf16", 1.0, 2.0 ** -8, 1.0),                          # tie, even is 1.0
        ("bf16", 1.0, 3 * 2.0 ** -8, 1.015625),                 # tie between 1+2^-7 and 1+2^-6
        ("bf16", 1.0, 2.0 ** -8 + 2.0 ** -20, 1.0078125),       # just above the tie
        ("f16", 1.0, 2.0 ** -11, 1.0),
        ("f16", 1.0, 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),
        ("f32", 1.0, 2.0 ** -24, 1.0),
        ("f32", 1.0, 3 * 2.0 ** -24, 1.0 + 2.0 ** -22),
        ("bf16", 2.0 ** 100, 2.0 ** -100, 2.0 ** 100),          # beyond float64's exact sum
        ("f16", 65504.0, 16.0, np.inf),                         # rounds past the largest f16
    ]
    for dt, xv, rv, hv in cases:
        h, f = o.forward_residual(np.array([[xv]]), np.array([[rv]]), [1.0], [1.0], [0.0], dt)
        assert h[0, 0] == hv, (dt, xv, rv, h[0, 0], hv)
        if np.isfinite(hv):
            assert math.isclose(f.y[0, 0], math.tanh(hv), rel_tol=1e-14)


def pin_residual_backward_composition(o):
    """dh = dres + dx: dres = 0 gives dx, dy = 0 gives dres with zero grads,
    and central differences of L(h) = sum(dres*h) + sum(dy*y(h)) give dh."""
    rng = np.random.default_rng(23)
    h = rng.standard_normal((3, 4))
    dy = rng.standard_normal((3, 4))
    dres = rng.standard_normal((3, 4))
    g, b, a = 1 + rng.standard_normal(4) * 0.1, rng.standard_normal(4) * 0.1, 0.8
    dh0, bw0, _ = o.backward_residual(h, dy, np.zeros((3, 4)), [a], g)
    assert np.array_equal(dh0, o.backward(h, dy, [a], g).dx)
    dh1, bw1, sc1 = o.backward_residual(h, np.zeros((3, 4)), dres, [a], g)
    assert np.array_equal(dh1, dres) and np.array_equal(sc1, np.abs(dres))
    assert not bw1.dgamma.any() and not bw1.dbeta.any() and bw1.dalpha == 0.0
    dh, bw, _ = o.backward_residual(h, dy, dres, [a], g)
    assert np.array_equal(bw.dgamma, bw0.dgamma) and bw.dalpha == bw0.dalpha

    def loss(hh):
        return math.fsum((dres * hh).ravel()) + math.fsum((dy * (g * np.tanh(a * hh) + b)).ravel())
    eps = 1e-6
    for i in range(3):
        for j in range(4):
            hp, hm = h.copy(), h.copy()
            hp[i, j] += eps
            hm[i, j] -= eps
            fd = (loss(hp) - loss(hm)) / (2 * eps)
            assert math.isclose(dh[i, j], fd, rel_tol=1e-7, abs_tol=1e-8), (i, j, dh[i, j], fd)
    rows, cols = np.divmod(np.arange(12), 4)
    dhs, scs = o.backward_dh_at(h[rows, cols], dy[rows, cols], dres[rows, cols], cols, [a], g)
    assert np.array_equal(dhs, dh.reshape(-1))


PINS = [
    pin_alpha_zero_gives_beta, pin_unit_affine_is_library_tanh, pin_rational_points,
    pin_complex_step, pin_central_differences, pin_integer_sums_alpha_inf,
    pin_integer_sums_alpha_zero, pin_ieee_alpha_inf_table, pin_large_u_sech2_not_cancelled,
    pin_odd_symmetry, pin_bruteforce_sums, pin_empty, pin_sampled_matches_full,
    pin_residual_zero_branch, pin_residual_integer_sums, pin_residual_rounding_ties,
    pin_residual_backward_composition,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(O)


# ------------------------------------------------- planted mistakes
# Each mutant replaces one internal of the oracle with a plausible mistake.

def _mut_forward(fn):
    return {"forward_core": fn}


def _bw_variant(dx=None, tg=None, ta=None, tb=None):
    def core(x, dy, alpha, gamma):
        with np.errstate(invalid="ignore", over="ignore"):
            u = alpha * x
            t = np.tanh(u)
            c = np.cosh(u)
            s = 1.0 / (c * c)
            env = dict(x=x, dy=dy, a=alpha, g=gamma, t=t, s=s, u=u)
            rdx = dy * gamma * alpha * s if dx is None else dx(env)
            rtg = dy * t if tg is None else tg(env)
            rta = dy * gamma * x * s if ta is None else ta(env)
            rtb = dy if tb is None else tb(env)
        return rdx, rtg, rtb, rta
    return {"backward_core": core}


def _res_y_from_unrounded(x, r, alpha, gamma, beta, x_dtype):
    h = O.residual_sum(x, r, x_dtype)
    return h, O.forward(np.asarray(x, np.float64) + np.asarray(r, np.float64), alpha, gamma, beta)


def _res_h_difference(x, r, alpha, gamma, beta, x_dtype):
    h = C.rne(np.asarray(x, np.float64) - np.asarray(r, np.float64), x_dtype)
    return h, O.forward(h, alpha, gamma, beta)


def _res_dh_variant(fn):
    def bres(h, dy, dres, alpha, gamma, want_dh=True):
        res = O.backward(h, dy, alpha, gamma, want_dx=want_dh)
        d = np.asarray(dres, np.float64)
        return fn(d, res.dx), res, np.abs(d) + np.abs(res.dx)
    return {"backward_residual": bres}


MUTANTS = {
    "res_y_from_unrounded_h": {"forward_residual": _res_y_from_unrounded},
    "res_h_is_difference": {"forward_residual": _res_h_difference},
    "res_dh_without_dres": _res_dh_variant(lambda d, dx: dx),
    "res_dh_minus_dres": _res_dh_variant(lambda d, dx: dx - d),
    "res_dh_without_dx": _res_dh_variant(lambda d, dx: d + 0 * dx),
    "fwd_alpha_dropped": _mut_forward(lambda x, a, g, b: g * np.tanh(x) + b),
    "fwd_beta_sign": _mut_forward(lambda x, a, g, b: g * np.tanh(a * x) - b),
    "fwd_gamma_beta_swapped": _mut_forward(lambda x, a, g, b: b * np.tanh(a * x) + g),
    "fwd_alpha_outside": _mut_forward(lambda x, a, g, b: g * a * np.tanh(x) + b),
    "sech2_unsquared": {"_sech2": lambda u: 1.0 / np.cosh(u)},
    "sech2_as_1_minus_t2": {"_sech2": lambda u: 1.0 - np.tanh(u) ** 2},
    "sech2_as_1_minus_t": {"_sech2": lambda u: 1.0 - np.abs(np.tanh(u))},
    "dx_alpha_dropped": _bw_variant(dx=lambda e: e["dy"] * e["g"] * e["s"]),
    "dx_gamma_dropped": _bw_variant(dx=lambda e: e["dy"] * e["a"] * e["s"]),
    "dx_sign": _bw_variant(dx=lambda e: -e["dy"] * e["g"] * e["a"] * e["s"]),
    "dx_uses_tanh": _bw_variant(dx=lambda e: e["dy"] * e["g"] * e["a"] * (1 - e["t"])),
    "dgamma_uses_sech2": _bw_variant(tg=lambda e: e["dy"] * e["s"]),
    "dgamma_times_gamma": _bw_variant(tg=lambda e: e["dy"] * e["t"] * e["g"]),
    "dalpha_gamma_dropped": _bw_variant(ta=lambda e: e["dy"] * e["x"] * e["s"]),
    "dalpha_from_dx": _bw_variant(ta=lambda e: e["dy"] * e["g"] * e["a"] * e["s"] * e["x"] / e["a"]),
    "dalpha_x_dropped": _bw_variant(ta=lambda e: e["dy"] * e["g"] * e["s"]),
    "dbeta_times_t": _bw_variant(tb=lambda e: e["dy"] * e["t"]),
    "gamma_transposed": _bw_variant(
        dx=lambda e: e["dy"] * np.resize(e["g"], e["dy"].shape[::-1]).T * e["a"] * e["s"]
        if e["dy"].ndim == 2 else e["dy"] * e["g"] * e["a"] * e["s"]),
}


def _run_pins_on(monkeypatch, patch):
    failed = []
    with monkeypatch.context() as m:
        for name, val in patch.items():
            m.setattr(O, name, val)
        for pin in PINS:
            try:
                pin(O)
            except (AssertionError, ValueError, IndexError, TypeError):
                failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(monkeypatch, mutant):
    failed = _run_pins_on(monkeypatch, MUTANTS[mutant])
    assert failed, f"no pin catches the planted mistake {mutant!r}"


# ------------------------------------------------- rounding and checkers

def test_rne_bf16_matches_torch_for_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(10)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38, 3.4e38, 1e-39, 2.0 ** -133,
                  2.0 ** -134, 3 * 2.0 ** -134, np.inf, -np.inf], dtype=np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = C.rne_bf16(v.astype(np.float64))
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.array_equal(got, want)


def test_rne_bf16_ties_and_direct_rounding():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins -> 1
    assert C.rne_bf16(1 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 ties between 1+2^-7 (odd) and 1+2^-6 (even) -> 1+2^-6
    assert C.rne_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    # just above the tie (not representable in float32) rounds up
    assert C.rne_bf16(1 + 2.0 ** -8 + 2.0 ** -40) == 1 + 2.0 ** -7
    assert C.rne_bf16(2.0 ** 128 * (1 - 2.0 ** -9)) == np.inf
    assert np.isnan(C.rne_bf16(np.nan))
    assert C.rne_bf16(2.0 ** -134) == 0.0            # tie at half the subnormal spacing
    assert C.rne_bf16(3 * 2.0 ** -134) == 2.0 ** -132


def test_ulp_bf16():
    assert C.ulp_bf16(1.0) == 2.0 ** -7
    assert C.ulp_bf16(1.99) == 2.0 ** -7
    assert C.ulp_bf16(2.0) == 2.0 ** -6
    assert C.ulp_bf16(-0.75) == 2.0 ** -8
    assert C.ulp_bf16(0.0) == 2.0 ** -133
    assert C.ulp_bf16(2.0 ** -127) == 2.0 ** -133


def test_checkers_accept_and_reject():
    ref = np.array([1.0, -2.0, 0.5, np.nan])
    ok = C.check_y(ref + np.array([1e-7, 0, 0, 0]), ref, np.abs(ref) + 0.1, "f32")
    assert ok.ok, ok
    bad = C.check_y(ref + np.array([1e-5, 0, 0, 0]), ref, np.abs(ref) + 0.1, "f32")
    assert bad.n_fail == 1
    nanbad = C.check_y(np.array([1.0, -2.0, np.nan, 1.0]), ref, np.abs(ref), "f32")
    assert nanbad.nan_mismatch == 2
    # bf16: one ulp is accepted, two are not
    r = np.array([1.5])
    assert C.check_y(r + 2.0 ** -7, r, r, "bf16").ok
    assert not C.check_y(r + 2.0 ** -6, r, r, "bf16").ok
    # condition-scaled: a cancelled y near 0 is compared at |gamma t| + |beta|
    assert C.check_y(np.array([1e-7]), np.array([0.0]), np.array([0.2]), "f32").ok
    # grads: relative to max(|g|, rss)
    assert C.check_grad([10.00001], [10.0], [1.0], "f32").ok
    assert not C.check_grad([10.001], [10.0], [1.0], "f32").ok
    assert C.check_grad([1e-3], [0.0], [1000.0], "f32").ok
    assert not C.check_dx(np.array([np.inf]), np.array([1.0]), "f32").ok


def test_checkers_accept_2d_bounds():
    ref = np.arange(12, dtype=np.float64).reshape(3, 4) + 1
    rep = C.check_y(ref.copy(), ref, np.abs(ref), "f32")
    assert rep.ok and rep.n == 12
    rep = C.check_dx(ref * (1 + 1e-5), ref, "f32", np.ones((3, 4)))
    assert rep.n_fail == 12


def test_rne_f16_matches_torch_for_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    v = np.concatenate([
        (rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000)).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504.0, 65519.0, 65520.0,
                  2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 6e-8, np.inf, -np.inf], dtype=np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.float16).to(torch.float64).numpy()
    got = C.rne_f16(v.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_rne_f16_direct_rounding_and_ulp():
    assert C.rne_f16(1 + 2.0 ** -11) == 1.0                      # tie to even
    assert C.rne_f16(1 + 2.0 ** -11 + 2.0 ** -40) == 1 + 2.0 ** -10
    assert C.rne_f16(65520.0) == np.inf and C.rne_f16(65519.99) == 65504.0
    assert C.rne_f16(2.0 ** -25) == 0.0 and C.rne_f16(3 * 2.0 ** -25) == 2.0 ** -23
    assert C.ulp_f16(1.0) == 2.0 ** -10 and C.ulp_f16(0.0) == 2.0 ** -24
    assert C.ulp_f16(2.0 ** -15) == 2.0 ** -24 and C.ulp_f16(1000.0) == 0.5
