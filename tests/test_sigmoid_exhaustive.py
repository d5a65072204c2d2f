"""Every float32 input of the device sigmoid, on the CPU.

The host build of the device's correctly rounded sigmoid (the same source
the kernels compile, ``sigmoid_cr.h``, built into ``libdspark_hostcheck.so``)
is run over every float32 x in (-104, 17.5) and compared bit for bit with
the oracle's ``sigmoid32``. Outside that range the value is a constant: 0
at and below -104 (sigmoid(-104) = 6.8e-46 is below half the smallest
subnormal, 7.0e-46), 1 at and above 17.5 (1 - sigmoid(17.5) = 2.5e-8 is
below half an ulp under 1), checked at a few points. The number of inputs
that take the double-double slow path is reported (1355).

The sigmoid decides every survival bit, and hence every verify length
("DSpark 自适应 Verify 怎样分配候选预算" §二, the runtime STS formula
sigmoid(z / T)).
"""

import multiprocessing as mp
import os
import sys
from pathlib import Path

import numpy as np
import pytest

ROOT = Path(__file__).resolve().parents[1]
CHUNK = 1 << 24
NEG = (0x80000000, 0xC2D00000)  # -0 .. just above -104
POS = (0x00000000, 0x418C0000)  # +0 .. just below 17.5


def _check_range(args):
    start, stop = args
    sys.path.insert(0, str(ROOT))
    from dspark_verify_scheduling_amd import _lib
    from oracle.sigmoid import sigmoid32

    x = np.arange(start, stop, dtype=np.uint64).astype(np.uint32).view(np.float32)
    y = np.empty_like(x)
    slow = np.zeros(x.shape, np.uint8)
    _lib.hostcheck().dspark_hostcheck_sigmoid(x.ctypes.data, y.ctypes.data, slow.ctypes.data,
                                              x.size, 0)
    ref = sigmoid32(x)
    bad = np.flatnonzero(y.view(np.uint32) != ref.view(np.uint32))
    return x.size, int(bad.size), int(slow.sum()), [float(x[i]) for i in bad[:4]]


def _chunks(lo, hi):
    return [(s, min(s + CHUNK, hi)) for s in range(lo, hi, CHUNK)]


def test_device_sigmoid_every_float32_input():
    pytest.importorskip("ctypes")
    sys.path.insert(0, str(ROOT))
    from dspark_verify_scheduling_amd import _lib

    try:
        _lib.hostcheck()
    except OSError as e:  # the host build is made by build()
        pytest.skip(f"host check library not built: {e}")
    jobs = _chunks(*NEG) + _chunks(*POS)
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.map(_check_range, jobs, chunksize=1)
    n = sum(r[0] for r in res)
    bad = sum(r[1] for r in res)
    slow = sum(r[2] for r in res)
    examples = [v for r in res for v in r[3]][:8]
    assert n == (NEG[1] - NEG[0]) + (POS[1] - POS[0]) == 2_220_621_824
    print(f"\n{n} float32 inputs in (-104, 17.5); {slow} took the double-double path; "
          f"{bad} differ from the oracle")
    assert bad == 0, examples
    assert slow > 0


def test_device_sigmoid_constant_outside_the_swept_range():
    sys.path.insert(0, str(ROOT))
    from dspark_verify_scheduling_amd import _lib
    from oracle.sigmoid import sigmoid32

    try:
        _lib.hostcheck()
    except OSError as e:
        pytest.skip(f"host check library not built: {e}")
    x = np.array([-104.0, -110.0, -1e6, -3.4e38, -np.inf, 17.5, 18.0, 100.0, 3.4e38, np.inf],
                 np.float32)
    y = np.empty_like(x)
    _lib.hostcheck().dspark_hostcheck_sigmoid(x.ctypes.data, y.ctypes.data, None, x.size, 0)
    assert np.array_equal(y.view(np.uint32), sigmoid32(x).view(np.uint32))
    assert (y[:5] == 0).all() and (y[5:] == 1).all()
