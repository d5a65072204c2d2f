"""Pins for the oracle's correctly rounded float32 sigmoid.

The sigmoid is the STS runtime calibration ``c = sigmoid(z / T)``. Its pins
come from mathematics, not from a second copy of the formula:

* closed forms: sigmoid(0) = 1/2 and sigmoid(ln 3) = 3/4;
* a 60-digit ``decimal`` evaluation with an exact nearest-float32 search
  (an independent computation: the fast path uses libm ``exp`` in fp64);
* the identity sigmoid(-x) = 1 - sigmoid(x), monotonicity, and the
  saturation points where the real value is within half an ulp of 1 or 0;
* the Tiny workload's confidences, supplied as logits, come back.
"""

import math

import numpy as np
import pytest

from oracle.sigmoid import nearest_f32, sigmoid32, sigmoid_decimal


def test_zero_is_half():
    assert sigmoid32(np.float32(0.0)) == np.float32(0.5)
    assert sigmoid32(np.float32(-0.0)) == np.float32(0.5)


def test_closed_form_ln3():
    # sigmoid(ln 3) = 3/4; x = RN32(ln 3) is off by < 2**-24 relative, and
    # sigmoid' = 3/16 there, so the result is 0.75 or one of its neighbours
    x = np.float32(math.log(3.0))
    y = sigmoid32(x)
    ulp = np.spacing(np.float32(0.75))
    assert abs(float(y) - 0.75) <= float(ulp)


def test_special_values():
    xs = np.array([np.inf, -np.inf, np.nan, 17.5, 100.0, -104.0, -1e30, 1e30], dtype=np.float32)
    y = sigmoid32(xs)
    assert y[0] == 1.0 and y[1] == 0.0 and np.isnan(y[2])
    assert y[3] == 1.0 and y[4] == 1.0  # 1 - sigmoid < 2**-25 once x > 25 ln 2
    assert y[5] == 0.0 and y[6] == 0.0  # sigmoid(-104) < 2**-150 rounds to +0
    assert y[7] == 1.0


def test_saturation_thresholds_match_exact_rounding():
    # around x = 25 ln 2 the real value crosses the midpoint 1 - 2**-25
    xs = np.linspace(17.0, 17.6, 2001).astype(np.float32)
    fast = sigmoid32(xs)
    for x, f in zip(xs[::50], fast[::50]):
        assert f == nearest_f32(sigmoid_decimal(float(x)))


def test_subnormal_range_against_decimal():
    xs = np.array([-87.0, -90.0, -95.5, -100.0, -103.2, -103.9], dtype=np.float32)
    fast = sigmoid32(xs)
    for x, f in zip(xs, fast):
        assert f == nearest_f32(sigmoid_decimal(float(x)))
    assert 0.0 < fast[1] < np.finfo(np.float32).tiny  # e^-90 is a float32 subnormal


@pytest.mark.parametrize("seed", [0, 1])
def test_fast_path_equals_decimal_reference(seed):
    rng = np.random.default_rng(seed)
    xs = np.concatenate([
        rng.normal(0, 3, 600),
        rng.uniform(-30, 30, 300),
        rng.uniform(-0.01, 0.01, 100),
    ]).astype(np.float32)
    fast = sigmoid32(xs)
    exact = np.array([nearest_f32(sigmoid_decimal(float(x))) for x in xs], dtype=np.float32)
    assert np.array_equal(fast.view(np.uint32), exact.view(np.uint32))


def test_symmetry_and_monotonicity():
    rng = np.random.default_rng(7)
    xs = np.sort(rng.normal(0, 4, 20000).astype(np.float32))
    y = sigmoid32(xs)
    assert np.all(np.diff(y.astype(np.float64)) >= 0)
    yn = sigmoid32(-xs)
    # sigmoid(x) + sigmoid(-x) = 1 exactly in reals; each side is within half an
    # ulp of its real value
    err = np.abs(y.astype(np.float64) + yn.astype(np.float64) - 1.0)
    bound = 0.5 * (np.spacing(y).astype(np.float64) + np.spacing(yn).astype(np.float64))
    assert np.all(err <= bound + 1e-300)


def test_within_half_ulp_of_fp64():
    rng = np.random.default_rng(3)
    xs = rng.uniform(-20, 20, 50000).astype(np.float32)
    y = sigmoid32(xs).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-xs.astype(np.float64)))
    assert np.all(np.abs(y - ref) <= 0.5 * np.spacing(y.astype(np.float32)).astype(np.float64) * (1 + 1e-9))


def test_tiny_config_confidences_round_trip():
    c = np.array([0.9, 0.8, 0.7, 0.6, 0.5, 0.4, 0.3], dtype=np.float64)
    z = np.log(c / (1 - c)).astype(np.float32)
    y = sigmoid32(z)
    assert np.all(np.abs(y.astype(np.float64) - c) < 1e-7)
