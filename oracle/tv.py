"""Soft accept-rate oracle: ``a = 1 - TV(softmax(q), softmax(p))`` and its cumprod.

Test infrastructure only (see ``oracle/__init__.py``).

[Budget] §二 (DeepSpec training target): ``accept_rate = 1 - 0.5 *
sum |draft_probs - target_probs|`` with both distributions softmaxes of the
logits, and ``confidence_prefix_targets = accept_rate.cumprod``. Under
rejection sampling the same number is ``sum_x min(p(x), q(x))``. The oracle
computes both forms and asserts that they agree.

Readings: the draft distribution q for position k (the one that proposed
draft k) pairs with target row k-1, the row that predicts position k. Both
softmaxes are max-subtracted and evaluated in fp64. The result is clamped
to [0, 1], which rounding can leave by about 1e-16. The product runs left to
right in fp64.
"""

from __future__ import annotations

import numpy as np

from .accept import as_f32_rows


def softmax64(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - np.max(x))
    return e / np.sum(e)


def tv_pair(q_row, p_row, dtype: str = "f32") -> float:
    """Soft accept-rate of one (draft row, target row) pair."""
    u = softmax64(as_f32_rows(q_row[None, :], dtype)[0])
    v = softmax64(as_f32_rows(p_row[None, :], dtype)[0])
    a = 1.0 - 0.5 * float(np.sum(np.abs(u - v)))
    a_min = float(np.sum(np.minimum(u, v)))
    assert abs(a - a_min) <= 1e-12, (a, a_min)
    return min(max(a, 0.0), 1.0)


def tv_accept(B, gamma, q, p, dtype: str, pairs=None):
    """``q[B, gamma, V]`` draft logits and ``p[B, R, V]`` target logits (R >= gamma).

    Returns ``(a, S)`` as fp64 ``[B, gamma]``. With ``pairs`` (a list of (r, k)
    with k 1-based) only those entries of ``a`` are computed (NaN elsewhere)
    and S is not formed."""
    B, gamma = int(B), int(gamma)
    a = np.full((B, gamma), np.nan)
    todo = pairs if pairs is not None else [(r, k) for r in range(B) for k in range(1, gamma + 1)]
    for r, k in todo:
        a[r, k - 1] = tv_pair(q[r, k - 1], p[r, k - 1], dtype)
    if pairs is not None:
        return a, None
    S = np.empty_like(a)
    for r in range(B):
        acc = 1.0
        for k in range(gamma):
            acc = acc * a[r, k]
            S[r, k] = acc
    return a, S
