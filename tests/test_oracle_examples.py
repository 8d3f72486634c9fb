"""Pins for the oracle against the worked examples the pages print (CPU only).

Fixture: tests/golden/worked_examples.json (each entry names its page and
section).  The outlier experiment's protocol -- 4096 standard-normal values
from numpy's default_rng(0), the outlier planted at index 0 of the first
128-value tile, error measured on the other 4095 values -- is the reading
under which every printed number reproduces.
"""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))
T4 = O.fp8_decode_table(O.E4M3)


def test_scale_rule_worked_example_amax_3p2():
    g = GOLDEN["scale_amax_3p2"]
    s, sinv = O.scale_from_amax(np.float32(g["amax"]), 1.0, O.E4M3)
    assert s[0] == np.float32(g["scale"])
    v = np.float32(g["value"]) * s[0]
    assert round(float(v), 6) == g["scaled"]
    c = int(O.fp8_encode(np.array([v], dtype=np.float32), O.E4M3)[0])
    assert T4[c] == g["rounded"]
    back = float(T4[c]) / float(s[0])
    assert round(back, 5) == g["returned"]
    assert round(abs(back - g["value"]) / g["value"] * 100, 2) == g["error_pct"]


def test_exercise_2_scale_and_smallest_step():
    g = GOLDEN["exercise_2"]
    s, _ = O.scale_from_amax(np.float32(g["amax"]), 1.0, O.E4M3)
    assert s[0] == np.float32(g["scale"])
    # effective step near zero: the smallest subnormal divided by the scale
    step = T4[0x01] / float(s[0])
    assert abs(step - 2.0 ** -9 / 560.0) < 1e-18
    assert round(step, 9) == 3.488e-06


def _experiment(outlier: float, per_tile: bool):
    x = np.random.default_rng(0).standard_normal(4096)
    x[0] = outlier
    x32 = x.astype(np.float32)
    if per_tile:
        am = np.abs(x32).reshape(32, 128).max(axis=1)
        s, _ = O.scale_from_amax(am, 1.0, O.E4M3)
        s = np.repeat(s, 128)
    else:
        s, _ = O.scale_from_amax(np.abs(x32).max(), 1.0, O.E4M3)
        s = np.full(4096, s[0], dtype=np.float32)
    v = (x32 * s).astype(np.float32)
    c = O.fp8_encode(v, O.E4M3)
    back = T4[c] / s.astype(np.float64)
    o = slice(1, 4096)
    err = back[o] - x[o]
    rmse = np.sqrt(np.sum(err ** 2) / np.sum(x[o] ** 2)) * 100
    zeroed = np.mean((c[o] & 0x7F) == 0) * 100
    subnormal = np.mean((c[o] & 0x78) == 0) * 100
    return rmse, zeroed, subnormal, float(s[0]), x, c


def test_outlier_experiment_1e5():
    g = GOLDEN["outlier_1e5"]
    rmse, zeroed, subnormal, s, x, c = _experiment(g["outlier"], per_tile=False)
    assert round(s, 5) == g["scale"]
    assert round(rmse, 2) == g["per_tensor_rmse_pct"]
    assert round(zeroed, 2) == g["zeroed_pct"]
    assert round(subnormal, 2) == g["subnormal_pct"]
    # "any value below about 0.22 rounds to zero": the flush threshold is half
    # the smallest subnormal divided by the scale
    thr = T4[0x01] / 2 / s
    assert round(thr, 2) == g["flush_threshold_about"]
    o = np.arange(1, 4096)
    z = (c[o] & 0x7F) == 0
    assert np.all(z[np.abs(x[o]) < 0.99 * thr]) and not np.any(z[np.abs(x[o]) > 1.01 * thr])
    rmse_t, *_ = _experiment(g["outlier"], per_tile=True)
    assert round(rmse_t, 2) == g["per_tile_rmse_pct"]


def test_outlier_experiment_1e4_zeroed():
    g = GOLDEN["outlier_1e4"]
    _, zeroed, *_ = _experiment(g["outlier"], per_tile=False)
    assert round(zeroed, 2) == g["zeroed_pct"]


@pytest.mark.parametrize("outlier", GOLDEN["rmse_floor"]["outliers_below"])
def test_rmse_floor_about_2p6_for_moderate_outliers(outlier):
    floor = GOLDEN["rmse_floor"]["floor_pct_about"]
    for per_tile in (False, True):
        rmse, *_ = _experiment(outlier, per_tile)
        assert abs(rmse - floor) < 0.2, (outlier, per_tile, rmse)


def test_per_tile_damage_confined_to_outlier_tile():
    # "Per-tile scaling confines the damage to the single tile that holds the outlier"
    x = np.random.default_rng(0).standard_normal(4096)
    clean = x.copy()
    x[0] = 1e5
    for arr, name in ((x, "outlier"), (clean, "clean")):
        x32 = arr.astype(np.float32)
        am = np.abs(x32).reshape(32, 128).max(axis=1)
        s, _ = O.scale_from_amax(am, 1.0, O.E4M3)
        v = (x32 * np.repeat(s, 128)).astype(np.float32)
        if name == "outlier":
            c_out = O.fp8_encode(v, O.E4M3)
        else:
            c_clean = O.fp8_encode(v, O.E4M3)
    assert np.array_equal(c_out[128:], c_clean[128:])
    assert not np.array_equal(c_out[:128], c_clean[:128])
