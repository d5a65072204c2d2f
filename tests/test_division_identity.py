"""The float32 quotient that the STS fitter's bin kernel forms as
RN32(z * RN64(1 / T)) equals the IEEE float32 quotient RN32(z / T).

The kernel evaluates one division per (record, candidate temperature) this
way. The argument: the double product is within 2^-52 (relative) of z / T,
while z / T is never a float32 rounding midpoint and lies more than 2^-49
(relative) from every one. Here numpy's IEEE float32 division is the
reference, over random bit patterns (every class: zeros, subnormals,
infinities, NaN), the fitter's temperature grids and significands close to
the hard cases.
"""

import numpy as np


def _mismatches(z, T):
    z = np.asarray(z, np.float32)
    T = np.asarray(T, np.float32)
    with np.errstate(all="ignore"):
        ref = z / T
        got = (z.astype(np.float64) * (1.0 / T.astype(np.float64))).astype(np.float32)
    same = (ref.view(np.uint32) == got.view(np.uint32)) | (np.isnan(ref) & np.isnan(got))
    return int((~same).sum())


def test_random_bit_patterns():
    rng = np.random.default_rng(11)
    n = 2_000_000
    z = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    T = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    assert _mismatches(z, T) == 0


def test_special_values():
    sp = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1.1754942e-38,
                   3.4028235e38, -3.4028235e38, 1.0, -1.0, 0.5, 3.0], np.float32)
    z, T = np.meshgrid(sp, sp)
    assert _mismatches(z.ravel(), T.ravel()) == 0


def test_temperature_grids_and_hard_significands():
    rng = np.random.default_rng(12)
    n = 1_000_000
    grid = np.exp(np.linspace(np.log(0.25), np.log(4.0), 64)).astype(np.float32)
    z = rng.normal(0, 4, n).astype(np.float32)
    assert _mismatches(z, grid[rng.integers(0, 64, n)]) == 0
    lo = (1 + rng.integers(0, 2**23, n) / 2**23).astype(np.float32)
    hi = (2 - rng.integers(1, 2**10, n) / 2**23).astype(np.float32)
    assert _mismatches(lo, hi) == 0 and _mismatches(hi, lo) == 0
