"""The offline tile tuner (bwd_dyt_forward_amd/tune.py): the committed tile
table is exactly what the tuner emits from the committed measurement record,
and the per-row choice rule (adopt at 3% better on the mean, guard at 3%
slower at any shape, then the fastest slowest shape) on synthetic ratios."""
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bwd_dyt_forward_amd")


@pytest.fixture(scope="module")
def tune():
    spec = importlib.util.spec_from_file_location("dyt_tune", os.path.join(PKG, "tune.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


RECORD = os.path.join(PKG, "tune_results.json")


def test_table_is_emitted_from_the_committed_record(tune):
    with open(tune.TABLE) as f:
        committed = f.read()
    assert tune.emit_text(RECORD) == committed


def test_record_covers_every_candidate_shape_and_kernel(tune):
    with open(RECORD) as f:
        data = json.load(f)
    assert set(data["candidates"]) == set(tune.CANDIDATES)
    assert data["default"] == tune.DEFAULT
    shapes = {(r["dtype"], r["M"], r["N"]) for r in data["results"]}
    want = {(d, M, N) for d, _, _, _, M, N, _ in tune._shapes()}
    assert shapes == want
    for r in data["results"]:
        for name in tune.CANDIDATES:
            t = r["us"][name]
            assert set(t) == {"fwd", "bwd", "rfwd"} and all(v > 0 for v in t.values())


def test_workloads_represent_the_rows_they_fall_in(tune):
    """100,003 x 255 float32 (2.55e7 elements) is a representative of the
    float32 161-512 row for 2^24 .. 2^26 elements, next to the two ends."""
    with open(tune.TABLE) as f:
        rows = [ln for ln in f if ln.lstrip().startswith("{DYT_F32, 161, 512, 16777216,")]
    assert len(rows) == 1
    assert "65793x255 263172x255 100003x255:" in rows[0]


def _reps(ratios, default="a", key="fwd"):
    """Representative shapes whose candidate times are the given ratios to a
    default time of 10 us."""
    n = len(next(iter(ratios.values())))
    reps = []
    for i in range(n):
        us = {default: {key: 10.0}}
        for name, r in ratios.items():
            us[name] = {key: 10.0 * r[i]}
        reps.append({"us": us})
    return reps


def test_choice_prefers_the_fastest_slowest_shape_over_the_best_mean(tune):
    # x has the better mean (0.85) but its slower end ties the default;
    # y is 10% better at its slower end
    ratios = {"x": [0.70, 1.00], "y": [0.88, 0.90]}
    reps = _reps(ratios)
    best, r = tune._choose(reps, ["a", "x", "y"], "a", "fwd")
    assert best == "y" and r == pytest.approx([0.88, 0.90])


def test_choice_guards_and_adopts(tune):
    # z is 3.5% slower at one shape (guard 3%); w is only 1.5% better on the
    # mean (adopt at 3%): neither replaces the default
    reps = _reps({"z": [0.50, 1.035], "w": [0.98, 0.99]})
    best, r = tune._choose(reps, ["a", "z", "w"], "a", "fwd")
    assert best == "a" and r == pytest.approx([1.0, 1.0])
    # just inside both thresholds a candidate qualifies
    reps = _reps({"z": [0.90, 1.029]})
    assert tune._choose(reps, ["a", "z"], "a", "fwd")[0] == "z"
    # ties on the slowest shape go to the better mean
    reps = _reps({"p": [0.95, 0.90], "q": [0.80, 0.90]})
    assert tune._choose(reps, ["a", "p", "q"], "a", "fwd")[0] == "q"
