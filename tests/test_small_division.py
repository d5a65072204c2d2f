"""The integer division that the planner and the pack kernels form as
trunc(RN32(n * RN32((1 + 2^-22) / d))) equals n // d for every 0 <= n < 2^15
and 1 <= d <= 65 (gamma <= 64 positions, gamma + 1 <= 65 verify slots per
request, at most 2 * 8192 slots). Exhaustive over that range; numpy's float32
division and multiplication are IEEE round-to-nearest, as the kernels' are.
"""

import numpy as np


def test_small_division_exhaustive():
    n = np.arange(1 << 15, dtype=np.int64)
    nf = n.astype(np.float32)
    for d in range(1, 66):
        inv = np.float32(1.0 + 2.0**-22) / np.float32(d)
        q = (nf * inv).astype(np.int64)  # float32 product, truncated
        assert np.array_equal(q, n // d), d


def test_plain_reciprocal_fails():
    # the 2^-22 margin matters: RN32(1 / d) alone truncates some exact
    # multiples to q - 1
    n = np.arange(1 << 15, dtype=np.int64)
    nf = n.astype(np.float32)
    bad = 0
    for d in range(1, 66):
        q = (nf * (np.float32(1.0) / np.float32(d))).astype(np.int64)
        bad += int((q != n // d).sum())
    assert bad > 0
