"""Pins for the STS fitter oracle.

Fixed by the pages' ECE definition on a hand-worked example, by a
construction whose labels match the survivals of one grid temperature
(zero calibration error there, large elsewhere), by the z / T invariance
(scaling the confidence logits and the grid by the same power of two changes
nothing), by the tie rule on perfectly calibrated data, and by the sequential
structure (position k is fitted on the survival already fitted for 1..k-1;
later positions never change earlier choices).
"""

import numpy as np
import pytest

import oracle
from oracle import sts


def test_ece_hand_example():
    # bins [0, .5) and [.5, 1]: |1 - 0.375| + |2 - 1.625| = 1.0 over 4 records
    S = np.array([0.125, 0.25, 0.75, 0.875], np.float32)
    y = np.array([0, 1, 1, 1])
    count, labels, conf, err = sts.ece_terms(S, y, 2)
    assert count.tolist() == [2, 2] and labels.tolist() == [1, 2]
    assert conf.tolist() == [int(0.375 * 2**40), int(1.625 * 2**40)]
    assert err == 2**40  # n * ECE = 1.0, so ECE = 0.25
    # over-confidence in one bin does not cancel under-confidence in another:
    # |2 - 0.375| + |0 - 1.625| = 3.25
    assert sts.ece_terms(S, np.array([1, 1, 0, 0]), 2)[3] == int(3.25 * 2**40)
    # 0.5 and 1.0 fall in the last bin
    assert sts.ece_terms(np.array([0.5, 1.0], np.float32), np.array([1, 1]), 2)[0].tolist() == [0, 2]
    # Brier: (0.125^2 + 0.75^2 + 0.25^2 + 0.125^2) / 4
    b = sts.brier_fx(S, y) / 2**40 / 4
    assert abs(b - (0.015625 + 0.5625 + 0.0625 + 0.015625) / 4) < 1e-12


def _calibrated_records(rng, t_true, probs, per_group):
    """Groups of records whose logit z = t_true * logit(p) and whose labels
    hit exactly round(p * per_group) positives."""
    z, y = [], []
    for p in probs:
        zz = np.float32(t_true * np.log(p / (1 - p)))
        pos = int(round(p * per_group))
        z += [zz] * per_group
        y += [1] * pos + [0] * (per_group - pos)
    order = rng.permutation(len(z))
    return np.array(z, np.float32)[order], np.array(y)[order]


def test_labels_matching_one_temperature_select_it():
    rng = np.random.default_rng(1)
    z1, y1 = _calibrated_records(rng, 2.0, [0.15, 0.35, 0.55, 0.85], 20)
    grid = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0], np.float32)
    out = sts.sts_fit(z1[:, None], y1[:, None], grid, 10)
    assert out["temps"].tolist() == [2.0] and out["t_index"].tolist() == [3]
    assert out["ece"][0] < 1e-6  # only the rounding of the sigmoid is left
    assert np.all(out["ece_fx"][0, [0, 1, 4, 5]] > 1000 * out["ece_fx"][0, 3])


def test_second_position_is_fitted_on_the_first_survival():
    # position 1: z = 0, so S_1 = sigmoid(0) = 0.5 at every T and half of every
    # group survives it (perfectly calibrated at any T: the first candidate
    # wins the tie). Position 2: within each group of 50, round(50 * 0.5 * c)
    # of the position-1 survivors survive again, c = sigmoid(z_2 / 1.5).
    n = 200
    z = np.zeros((n, 2), np.float32)
    y = np.zeros((n, 2), np.int64)
    for g, c in enumerate([0.3, 0.7, 0.9, 0.5]):
        rows = np.arange(g * 50, (g + 1) * 50)
        z[rows, 1] = np.float32(1.5 * np.log(c / (1 - c)))
        y[rows[:25], 0] = 1
        y[rows[: int(round(50 * 0.5 * c))], 1] = 1
    assert np.all(y[:, 1] <= y[:, 0])
    grid = np.array([0.75, 1.5, 3.0], np.float32)
    out = sts.sts_fit(z, y, grid, 20)
    assert out["t_index"].tolist() == [0, 1]
    assert out["ece_fx"][0].tolist() == [0, 0, 0]
    one = sts.sts_fit(z[:, :1], y[:, :1], grid, 20)
    assert one["t_index"][0] == out["t_index"][0]  # later positions do not move it
    # position 2 multiplied the fitted S_1 = 0.5
    assert np.all(out["survival"][:, 0] == np.float32(0.5))
    expect = (np.float32(0.5) * oracle.sigmoid32(z[:, 1] / grid[1])).astype(np.float32)
    assert np.array_equal(out["survival"][:, 1], expect)


@pytest.mark.parametrize("seed", range(5))
def test_invariant_under_common_power_of_two_scaling(seed):
    rng = np.random.default_rng(10 + seed)
    n, g = 300, 4
    z = rng.normal(1.0, 2.0, (n, g)).astype(np.float32)
    y = np.cumprod(rng.random((n, g)) < 0.7, axis=1).astype(np.int64)
    grid = np.array([0.5, 0.8, 1.0, 1.3, 2.0, 3.1], np.float32)
    a = sts.sts_fit(z, y, grid, 15)
    b = sts.sts_fit(z * 8, y, grid * 8, 15)
    assert np.array_equal(a["t_index"], b["t_index"])
    assert np.array_equal(a["survival"], b["survival"])
    assert np.array_equal(a["ece_fx"], b["ece_fx"])
    # the chosen candidate has the smallest error, the first among equals
    for k in range(g):
        row = a["ece_fx"][k]
        assert a["t_index"][k] == int(np.argmin(row))


def test_perfectly_calibrated_ties_take_the_first_candidate():
    z = np.zeros((8, 1), np.float32)  # sigmoid(0 / T) = 0.5 for every T
    y = np.array([[1], [0]] * 4)
    out = sts.sts_fit(z, y, np.array([3.0, 1.0, 2.0], np.float32), 4)
    assert out["ece_fx"].tolist() == [[0, 0, 0]]
    assert out["t_index"].tolist() == [0] and out["temps"].tolist() == [3.0]
    assert out["brier"][0] == 0.25


def test_nan_survival_bins_like_zero():
    # a NaN logit makes its survival NaN from that position on; it is binned
    # and summed as 0, exactly like a -inf logit (whose survival is 0)
    rng = np.random.default_rng(4)
    n, g = 400, 3
    z = rng.normal(0.5, 2.0, (n, g)).astype(np.float32)
    y = np.cumprod(rng.random((n, g)) < 0.6, axis=1).astype(np.int64)
    y[[7, 19, 30], :] = 0
    grid = np.array([0.5, 1.0, 2.0, 4.0], np.float32)
    zn, zi = z.copy(), z.copy()
    zn[7, 0] = zn[19, 1] = zn[30, 2] = np.nan
    zi[7, 0] = zi[19, 1] = zi[30, 2] = -np.inf
    a, b = sts.sts_fit(zn, y, grid, 10), sts.sts_fit(zi, y, grid, 10)
    assert np.array_equal(a["ece_fx"], b["ece_fx"])
    assert np.array_equal(a["t_index"], b["t_index"]) and np.array_equal(a["brier"], b["brier"])
    assert np.isnan(a["survival"][7]).all() and (b["survival"][7] == 0).all()
    assert np.isnan(a["survival"][19, 1:]).all() and not np.isnan(a["survival"][19, 0])
    # and a NaN that counted as anything else would move the error
    assert sts.ece_terms(np.array([np.nan], np.float32), np.array([0]), 4)[3] == 0
