"""Accept/reject pins of the tolerance checkers in oracle/compare.py.

The checkers turn the stated tolerances into pass/fail decisions for every
parity test, so each branch is pinned at its boundary: an error just inside
the stated bound must pass and one just beyond it must fail. The bounds
themselves are the dtype contract of the Liger-Kernel pull request
"fix(dyt): use a 1D grid and tile small-width rows" (Summary, "Precision":
y and dx in x's dtype, parameter gradients in the parameters' dtype with
float32 accumulation), made numeric as float32 rel 1e-6 on y and dx, one
unit in the last place of the rounded oracle for 2-byte outputs, rel 1e-5
for the float32-accumulated gradients. The expected decisions below are
worked out by hand from those figures, with the unit in the last place
written as a power of two (bfloat16 keeps 8 significant bits, float16 11),
not computed by the checkers' own helpers.

``test_checker_pins_catch_planted_mistakes`` replaces one checker (or one
of its helpers) at a time with a plausibly loosened or mis-scaled version
and asserts that at least one pin fails.
"""
import numpy as np
import pytest

from oracle import compare as C

F32_TINY = 2.0 ** -149


def _ok(rep):
    assert rep.ok, str(rep)


def _bad(rep, n_fail=None):
    assert not rep.ok, f"should have failed: {rep}"
    if n_fail is not None:
        assert rep.n_fail == n_fail, str(rep)


# ------------------------------------------------------------------ pins
# Each pin takes the compare module and raises AssertionError on failure.

def pin_y_f32(c):
    ref = np.array([1.0, -0.5, 0.0])
    scale = np.array([1.25, 0.75, 0.5])          # |gamma t| + |beta|
    _ok(c.check_y(ref + 0.999e-6 * scale, ref, scale, "f32"))
    _ok(c.check_y(ref - 0.999e-6 * scale, ref, scale, "f32"))
    _bad(c.check_y(ref + np.array([1.001e-6 * 1.25, 0, 0]), ref, scale, "f32"), 1)
    # a cancelled y (0) is judged at its scale, not at |y| = 0
    _bad(c.check_y(np.array([0.0, 0.0, 0.5 * 1.01e-6]), ref * 0, scale, "f32"), 1)


def pin_y_bf16(c):
    r = np.array([1.5])                           # ulp(1.5) = 2^-7 in bfloat16
    _ok(c.check_y(r + 2.0 ** -7, r, r, "bf16"))
    _bad(c.check_y(r + 2.0 ** -6, r, r, "bf16"))
    # near-cancelling y: one ulp at the scale 1.5, not at |y| = 2^-20
    _ok(c.check_y(np.array([2.0 ** -7]), np.array([2.0 ** -20]), r, "bf16"))
    _bad(c.check_y(np.array([2.0 ** -6]), np.array([2.0 ** -20]), r, "bf16"))
    # the error is taken from the rounded oracle: y* = 1 + 0.4 * 2^-7 rounds
    # to 1, and 1 - 2^-7 is one ulp (2^-7 at 1.003) from it, though 1.4 ulp
    # from y* itself
    ys = np.array([1.0 + 0.4 * 2.0 ** -7])
    _ok(c.check_y(np.array([1.0 - 2.0 ** -7]), ys, ys, "bf16"))
    _bad(c.check_y(np.array([1.0 + 2.0 ** -6]), ys, ys, "bf16"))
    # bfloat16 overflows only past 2^128
    _ok(c.check_y(np.array([3.0e38]), np.array([3.0e38]), np.array([3.0e38]), "bf16"))


def pin_y_f16(c):
    r = np.array([1.5])                           # ulp(1.5) = 2^-10 in float16
    _ok(c.check_y(r + 2.0 ** -10, r, r, "f16"))
    _bad(c.check_y(r + 2.0 ** -9, r, r, "f16"))
    ys = np.array([1.0 + 0.4 * 2.0 ** -10])       # rounds to 1 in float16
    _ok(c.check_y(np.array([1.0 - 2.0 ** -10]), ys, ys, "f16"))
    # float16 subnormals: spacing 2^-24
    s = np.array([3.0 * 2.0 ** -24])
    _ok(c.check_y(s + 2.0 ** -24, s, s, "f16"))
    _bad(c.check_y(s + 2.0 ** -23, s, s, "f16"))
    # 65520 rounds past the largest float16 (65504) to +inf
    big = np.array([65520.0])
    _ok(c.check_y(np.array([np.inf]), big, big, "f16"))
    _bad(c.check_y(np.array([65504.0]), big, big, "f16"))


def pin_dx_f32(c):
    ref = np.array([2.0, -3.0e-3])
    _ok(c.check_dx(ref * (1 + 0.999e-6), ref, "f32"))
    _bad(c.check_dx(ref * (1 + 1.001e-6), ref, "f32"), 2)
    # dx is a product, judged at |dx*| alone: rel 1e-6 of 1e-30 is 1e-36
    tiny = np.array([1e-30])
    _bad(c.check_dx(tiny * (1 + 2e-6), tiny, "f32"), 1)
    # underflow floor: 2^-149 (1 + 4 |dy gamma alpha|)
    z = np.array([0.0])
    _ok(c.check_dx(np.array([13 * F32_TINY]), z, "f32", np.array([3.0])))
    _bad(c.check_dx(np.array([14 * F32_TINY]), z, "f32", np.array([3.0])))
    _ok(c.check_dx(np.array([F32_TINY]), z, "f32"))
    _bad(c.check_dx(np.array([2 * F32_TINY]), z, "f32"))


def _pin_dx_2byte(c, dt, ulp1, ulp_small):
    r = np.array([1.5])
    _ok(c.check_dx(r + ulp1, r, dt))
    _bad(c.check_dx(r + 2 * ulp1, r, dt))
    # no condition scale: 2^-10 is judged at its own ulp
    s = np.array([2.0 ** -10])
    _ok(c.check_dx(s + ulp_small, s, dt))
    _bad(c.check_dx(s + 2 * ulp_small, s, dt))
    # rounded oracle: dx* = 1 + 0.4 ulp rounds to 1
    ds = np.array([1.0 + 0.4 * ulp1])
    _ok(c.check_dx(np.array([1.0 - ulp1]), ds, dt))


def pin_dx_bf16(c):
    _pin_dx_2byte(c, "bf16", 2.0 ** -7, 2.0 ** -17)


def pin_dx_f16(c):
    _pin_dx_2byte(c, "f16", 2.0 ** -10, 2.0 ** -20)


def pin_grad_f32(c):
    _ok(c.check_grad([10.0 + 0.999e-4], [10.0], [1.0], "f32"))
    _bad(c.check_grad([10.0 + 1.001e-4], [10.0], [1.0], "f32"))
    # a random-sign sum near 0 is judged at its RSS
    _ok(c.check_grad([0.999e-2], [0.0], [1000.0], "f32"))
    _bad(c.check_grad([1.001e-2], [0.0], [1000.0], "f32"))
    # and a large total at its own size, even with a small RSS
    _ok(c.check_grad([1000.0 + 0.999e-2], [1000.0], [1.0], "f32"))
    _bad(c.check_grad([1000.0 + 1.001e-2], [1000.0], [1.0], "f32"))


def _pin_grad_2byte(c, dt, ulp3):
    # g* = 3: one ulp of the parameter dtype (bfloat16 2^-6, float16 2^-9)
    _ok(c.check_grad([3.0 + ulp3], [3.0], [0.0], dt))
    _bad(c.check_grad([3.0 + 2 * ulp3], [3.0], [0.0], dt))
    # plus 1e-5 of the RSS of the summed terms
    _ok(c.check_grad([0.999e-3], [0.0], [100.0], dt))
    _bad(c.check_grad([1.001e-3], [0.0], [100.0], dt))
    # rounded oracle: g* = 3 + 0.4 ulp rounds to 3
    _ok(c.check_grad([3.0 - ulp3], [3.0 + 0.4 * ulp3], [0.0], dt))


def pin_grad_bf16(c):
    _pin_grad_2byte(c, "bf16", 2.0 ** -6)


def pin_grad_f16(c):
    _pin_grad_2byte(c, "f16", 2.0 ** -9)


def pin_dh_f32(c):
    # dh = dres + dx cancelling to 0 is judged at |dres| + |dx*| = 2
    z = np.array([0.0])
    two = np.array([2.0])
    _ok(c.check_dh(np.array([1.999e-6]), z, two, "f32"))
    _bad(c.check_dh(np.array([2.001e-6]), z, two, "f32"))
    ref = np.array([1.0])
    _ok(c.check_dh(ref + 0.999e-6, ref, ref, "f32"))
    _bad(c.check_dh(ref + 1.001e-6, ref, ref, "f32"))
    # dx's underflow floor carries over
    _ok(c.check_dh(np.array([5 * F32_TINY]), z, z, "f32", np.array([1.0])))
    _bad(c.check_dh(np.array([6 * F32_TINY]), z, z, "f32", np.array([1.0])))


def _pin_dh_2byte(c, dt, ulp15, ulp3):
    z = np.array([0.0])
    s = np.array([1.5])
    _ok(c.check_dh(np.array([ulp15]), z, s, dt))
    _bad(c.check_dh(np.array([2 * ulp15]), z, s, dt))
    t = np.array([3.0])
    _ok(c.check_dh(t + ulp3, t, t, dt))
    _bad(c.check_dh(t + 2 * ulp3, t, t, dt))


def pin_dh_bf16(c):
    _pin_dh_2byte(c, "bf16", 2.0 ** -7, 2.0 ** -6)


def pin_dh_f16(c):
    _pin_dh_2byte(c, "f16", 2.0 ** -10, 2.0 ** -9)


def pin_exact(c):
    a = np.array([1.0, -0.0, np.nan, np.inf, 2.0 ** -149, -3.5])
    _ok(c.check_exact(a.copy(), a))
    _ok(c.check_exact(np.array([0.0]), np.array([-0.0])))     # values, not sign bits
    _bad(c.check_exact(np.array([np.nextafter(1.0, 2.0)]), np.array([1.0])), 1)
    _bad(c.check_exact(np.array([np.nextafter(np.float32(1), np.float32(2))], np.float64),
                       np.array([1.0])), 1)
    _bad(c.check_exact(np.array([2.0 ** -149]), np.array([0.0])), 1)
    _bad(c.check_exact(np.array([1.0]), np.array([np.nan])))
    _bad(c.check_exact(np.array([-np.inf]), np.array([np.inf])))


def pin_special_values(c):
    """NaN exactly where the oracle has NaN, infinities equal, every checker."""
    ref = np.array([1.0, np.nan, np.inf, -2.0])
    sc = np.abs(np.nan_to_num(ref, posinf=1.0)) + 1.0
    for dt in ("f32", "bf16", "f16"):
        calls = [
            lambda g: c.check_y(g, ref, sc, dt),
            lambda g: c.check_dx(g, ref, dt),
            lambda g: c.check_grad(g, ref, sc, dt),
            lambda g: c.check_dh(g, ref, sc, dt),
        ]
        for f in calls:
            _ok(f(ref.copy()))
            rep = f(np.array([np.nan, np.nan, np.inf, -2.0]))
            assert rep.nan_mismatch == 1, str(rep)
            rep = f(np.array([1.0, 5.0, np.inf, -2.0]))
            assert rep.nan_mismatch == 1, str(rep)
            rep = f(np.array([1.0, np.nan, -np.inf, -2.0]))
            assert rep.inf_mismatch == 1, str(rep)
            rep = f(np.array([1.0, np.nan, 3.0e38, -2.0]))
            assert rep.inf_mismatch == 1, str(rep)


def pin_report_counts(c):
    """n counts every element; 2-D inputs with per-element bounds."""
    ref = np.arange(1.0, 13.0).reshape(3, 4)
    rep = c.check_y(ref.copy(), ref, ref, "f32")
    assert rep.ok and rep.n == 12, str(rep)
    rep = c.check_dx(ref * (1 + 1e-5), ref, "f32", np.ones((3, 4)))
    assert rep.n_fail == 12, str(rep)


CHECKER_PINS = [
    pin_y_f32, pin_y_bf16, pin_y_f16, pin_dx_f32, pin_dx_bf16, pin_dx_f16,
    pin_grad_f32, pin_grad_bf16, pin_grad_f16, pin_dh_f32, pin_dh_bf16, pin_dh_f16,
    pin_exact, pin_special_values, pin_report_counts,
]


@pytest.mark.parametrize("pin", CHECKER_PINS, ids=lambda p: p.__name__)
def test_checker_pin(pin):
    pin(C)


# ------------------------------------------------------ planted mistakes
# Each mutant stands in for one function of the compare module; it is built
# from the original helpers so that only the named mistake differs.

_orig = {name: getattr(C, name) for name in
         ("check_y", "check_dx", "check_grad", "check_dh", "check_exact", "_finish",
          "ulp_f16", "ulp_bf16", "rne_f16", "rne")}


def _a(v):
    return np.asarray(v, dtype=np.float64)


def _wrap_dtype(fn_name, dt, replacement):
    """The original checker, except for dtype dt, where `replacement` runs."""
    orig = _orig[fn_name]

    def f(*args, **kw):
        args = list(args)
        # the dtype is the 4th positional argument of check_y/check_grad/check_dh
        # and the 3rd of check_dx
        pos = 2 if fn_name == "check_dx" else 3
        dtype = kw.get("dtype", args[pos] if len(args) > pos else None)
        if dtype == dt:
            return replacement(*args, **kw)
        return orig(*args, **kw)
    return f


def _y_scaled(k):
    return lambda got, y, s, dt, name="y": _orig["check_y"](got, y, _a(s) * k, dt, name)


CHECKER_MUTANTS = {
    # y
    "y_f32_rel_1e5": {"check_y": _wrap_dtype("check_y", "f32", _y_scaled(10.0))},
    "y_f32_value_scaled": {"check_y": _wrap_dtype(
        "check_y", "f32", lambda g, y, s, dt, name="y": _orig["check_y"](g, y, np.abs(_a(y)), dt, name))},
    "y_bf16_two_ulp": {"check_y": _wrap_dtype("check_y", "bf16", _y_scaled(2.0))},
    "y_bf16_ignores_scale": {"check_y": _wrap_dtype(
        "check_y", "bf16", lambda g, y, s, dt, name="y": C._finish(
            name, g, C.rne(y, dt), C.ulp(np.abs(_a(y)), dt)))},
    "y_bf16_unrounded_oracle": {"check_y": _wrap_dtype(
        "check_y", "bf16", lambda g, y, s, dt, name="y": C._finish(
            name, g, _a(y), C.ulp(np.maximum(np.abs(_a(y)), _a(s)), dt)))},
    "y_f16_as_bf16": {"check_y": _wrap_dtype(
        "check_y", "f16", lambda g, y, s, dt, name="y": _orig["check_y"](g, y, s, "bf16", name))},
    # dx
    "dx_f32_no_floor": {"check_dx": _wrap_dtype(
        "check_dx", "f32", lambda g, d, dt, k=None, name="dx": C._finish(name, g, d, 1e-6 * np.abs(_a(d))))},
    "dx_f32_floor_ignores_dga": {"check_dx": _wrap_dtype(
        "check_dx", "f32", lambda g, d, dt, k=None, name="dx": _orig["check_dx"](g, d, dt, None, name))},
    "dx_f32_rel_2e6": {"check_dx": _wrap_dtype(
        "check_dx", "f32", lambda g, d, dt, k=None, name="dx": C._finish(
            name, g, d, 2e-6 * np.abs(_a(d)) + F32_TINY))},
    "dx_bf16_two_ulp": {"check_dx": _wrap_dtype(
        "check_dx", "bf16", lambda g, d, dt, k=None, name="dx": C._finish(
            name, g, C.rne(d, dt), 2 * C.ulp(d, dt)))},
    "dx_bf16_unit_scale": {"check_dx": _wrap_dtype(
        "check_dx", "bf16", lambda g, d, dt, k=None, name="dx": C._finish(
            name, g, C.rne(d, dt), C.ulp(np.maximum(np.abs(_a(d)), 1.0), dt)))},
    "dx_bf16_unrounded_oracle": {"check_dx": _wrap_dtype(
        "check_dx", "bf16", lambda g, d, dt, k=None, name="dx": C._finish(name, g, d, C.ulp(d, dt)))},
    "dx_f16_two_ulp": {"check_dx": _wrap_dtype(
        "check_dx", "f16", lambda g, d, dt, k=None, name="dx": C._finish(
            name, g, C.rne(d, dt), 2 * C.ulp(d, dt)))},
    "dx_f16_as_bf16": {"check_dx": _wrap_dtype(
        "check_dx", "f16", lambda g, d, dt, k=None, name="dx": _orig["check_dx"](g, d, "bf16", k, name))},
    # gradients
    "grad_f32_no_rss": {"check_grad": _wrap_dtype(
        "check_grad", "f32", lambda g, r, rss, dt, name="grad": C._finish(
            name, np.atleast_1d(_a(g)), np.atleast_1d(_a(r)), 1e-5 * np.abs(np.atleast_1d(_a(r))) + F32_TINY))},
    "grad_f32_rss_only": {"check_grad": _wrap_dtype(
        "check_grad", "f32", lambda g, r, rss, dt, name="grad": C._finish(
            name, np.atleast_1d(_a(g)), np.atleast_1d(_a(r)), 1e-5 * np.atleast_1d(_a(rss)) + F32_TINY))},
    "grad_f32_rel_1e4": {"check_grad": _wrap_dtype(
        "check_grad", "f32", lambda g, r, rss, dt, name="grad": _orig["check_grad"](
            g, r, 10 * np.maximum(np.abs(_a(r)), _a(rss)), dt, name))},
    "grad_bf16_no_ulp": {"check_grad": _wrap_dtype(
        "check_grad", "bf16", lambda g, r, rss, dt, name="grad": C._finish(
            name, np.atleast_1d(_a(g)), C.rne(np.atleast_1d(_a(r)), dt), 1e-5 * np.atleast_1d(_a(rss))))},
    "grad_bf16_two_ulp": {"check_grad": _wrap_dtype(
        "check_grad", "bf16", lambda g, r, rss, dt, name="grad": C._finish(
            name, np.atleast_1d(_a(g)), C.rne(np.atleast_1d(_a(r)), dt),
            2 * C.ulp(np.atleast_1d(_a(r)), dt) + 1e-5 * np.atleast_1d(_a(rss))))},
    "grad_bf16_rss_1e4": {"check_grad": _wrap_dtype(
        "check_grad", "bf16", lambda g, r, rss, dt, name="grad": _orig["check_grad"](
            g, r, 10 * _a(rss), dt, name))},
    "grad_bf16_unrounded_oracle": {"check_grad": _wrap_dtype(
        "check_grad", "bf16", lambda g, r, rss, dt, name="grad": C._finish(
            name, np.atleast_1d(_a(g)), np.atleast_1d(_a(r)),
            C.ulp(np.atleast_1d(_a(r)), dt) + 1e-5 * np.atleast_1d(_a(rss))))},
    "grad_f16_as_bf16": {"check_grad": _wrap_dtype(
        "check_grad", "f16", lambda g, r, rss, dt, name="grad": _orig["check_grad"](g, r, rss, "bf16", name))},
    # dh of the residual backward
    "dh_f32_scale_x10": {"check_dh": _wrap_dtype(
        "check_dh", "f32", lambda g, d, s, dt, k=None, name="dh": _orig["check_dh"](g, d, 10 * _a(s), dt, k, name))},
    "dh_f32_no_floor": {"check_dh": _wrap_dtype(
        "check_dh", "f32", lambda g, d, s, dt, k=None, name="dh": C._finish(name, g, d, 1e-6 * _a(s)))},
    "dh_bf16_scale_x10": {"check_dh": _wrap_dtype(
        "check_dh", "bf16", lambda g, d, s, dt, k=None, name="dh": _orig["check_dh"](g, d, 10 * _a(s), dt, k, name))},
    "dh_bf16_ignores_scale": {"check_dh": _wrap_dtype(
        "check_dh", "bf16", lambda g, d, s, dt, k=None, name="dh": C._finish(
            name, g, C.rne(d, dt), C.ulp(np.abs(_a(d)), dt)))},
    "dh_f16_two_ulp": {"check_dh": _wrap_dtype(
        "check_dh", "f16", lambda g, d, s, dt, k=None, name="dh": _orig["check_dh"](g, d, 2 * _a(s), dt, k, name))},
    # exact comparison and the shared machinery
    "exact_one_ulp_slack": {"check_exact": lambda g, r, name="h": C._finish(
        name, g, r, np.spacing(np.abs(_a(r))))},
    "exact_float32_slack": {"check_exact": lambda g, r, name="h": C._finish(
        name, g, r, 2.0 ** -23 * np.abs(_a(r)))},
    "finish_ignores_nan": {"_finish": lambda name, g, r, b: _orig["_finish"](
        name, np.where(np.isnan(_a(g)) | np.isnan(_a(r)), 0.0, _a(g)),
        np.where(np.isnan(_a(g)) | np.isnan(_a(r)), 0.0, _a(r)), b)},
    "finish_ignores_inf_sign": {"_finish": lambda name, g, r, b: _orig["_finish"](
        name, np.where(np.isinf(_a(g)), np.abs(_a(g)), _a(g)),
        np.where(np.isinf(_a(r)), np.abs(_a(r)), _a(r)), b)},
    "finish_bound_1pct_loose": {"_finish": lambda name, g, r, b: _orig["_finish"](name, g, r, _a(b) * 1.01)},
    "ulp_f16_doubled": {"ulp_f16": lambda v: 2 * _orig["ulp_f16"](v)},
    "ulp_bf16_doubled": {"ulp_bf16": lambda v: 2 * _orig["ulp_bf16"](v)},
    "rne_f16_truncates": {"rne_f16": lambda v: np.where(
        np.isfinite(_a(v)), np.trunc(_a(v) * 2.0 ** 10) / 2.0 ** 10, _a(v))},
}


def _run_checker_pins(monkeypatch, patch):
    failed = []
    with monkeypatch.context() as m:
        for name, val in patch.items():
            m.setattr(C, name, val)
        for pin in CHECKER_PINS:
            try:
                pin(C)
            except (AssertionError, ValueError, IndexError, TypeError):
                failed.append(pin.__name__)
    return failed


def test_checker_pins_pass_unpatched(monkeypatch):
    assert _run_checker_pins(monkeypatch, {}) == []


@pytest.mark.parametrize("mutant", sorted(CHECKER_MUTANTS))
def test_checker_pins_catch_planted_mistakes(monkeypatch, mutant):
    failed = _run_checker_pins(monkeypatch, CHECKER_MUTANTS[mutant])
    assert failed, f"no checker pin catches the planted mistake {mutant!r}"
