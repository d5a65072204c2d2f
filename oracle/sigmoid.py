"""Correctly rounded float32 logistic sigmoid (oracle; test infrastructure only).

[Budget] §二 (STS, the runtime formula ``c_i = sigmoid(z_i / T_i)``) gives the
calibrated per-position confidence. The pages do not fix its precision. The
kernels and the oracle both take it as the float32 value nearest to the real
number ``1 / (1 + exp(-x))`` (round to nearest, ties to even), where
``x = RN32(z / T)``. That is a plain definition with a unique result, so the
survival values that decide ``verify_lens`` agree bit for bit on both sides.

Method: a vectorised fp64 evaluation whose relative error is far below
2**-40, then a rounding-band test. If ``y(1 - 2**-40)`` and ``y(1 + 2**-40)``
round to the same float32, the true value (inside that band) rounds there
too. Otherwise the value is recomputed with Python's ``decimal`` module at
60 significant digits (its ``exp`` is correctly rounded at that precision),
and the nearest float32 is picked by exact comparison with the neighbours.
"""

from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np

_BAND = 2.0 ** -40


def sigmoid_decimal(x: float) -> Decimal:
    """sigmoid(x) to 60 significant digits."""
    with localcontext() as ctx:
        ctx.prec = 60
        e = (-Decimal(float(x))).exp()
        return Decimal(1) / (Decimal(1) + e)


def nearest_f32(y: Decimal) -> np.float32:
    """The float32 nearest to the real number ``y`` (ties to even mantissa)."""
    f = np.float32(float(y))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def rank(c):
        return (abs(Decimal(float(c)) - y), int(np.asarray(c).view(np.uint32)) & 1)

    return np.float32(min(cands, key=rank))


def sigmoid32(x) -> np.ndarray:
    """Correctly rounded float32 sigmoid of float32 ``x`` (elementwise).

    NaN maps to NaN; -inf to 0; +inf to 1."""
    x = np.asarray(x, dtype=np.float32)
    xd = x.astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        y = 1.0 / (1.0 + np.exp(-xd))
        lo = (y * (1.0 - _BAND)).astype(np.float32)
        hi = (y * (1.0 + _BAND)).astype(np.float32)
    out = y.astype(np.float32)
    unsure = (lo != hi) & ~np.isnan(xd)
    if np.any(unsure):
        flat_out = out.reshape(-1)
        flat_x = x.reshape(-1)
        for i in np.flatnonzero(unsure.reshape(-1)):
            flat_out[i] = nearest_f32(sigmoid_decimal(float(flat_x[i])))
        out = flat_out.reshape(x.shape)
    return out
