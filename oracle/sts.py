"""Sequential temperature scaling (STS) fitter oracle. TEST INFRASTRUCTURE ONLY.

[Budget] §二 (runtime STS: c_i = sigmoid(z_i / T_i), S_k = prod_{i<=k} c_i;
the fitter searches a positive temperature per position, in order, keeping
the cumulative survival already fitted for the earlier positions, and picks
for the current position the candidate with the lower expected calibration
error against the greedy prefix label). [CSSD] "为什么置信度必须校准" (the
ECE over confidence bins, ECE = sum_b |I_b| / n * |acc(I_b) - conf(I_b)|,
and the label of position k only has its meaning given that positions
1..k-1 survived, so the cumulative survival is what is calibrated).

What it computes, for positions k = 1..gamma in order:
  for every candidate T of the grid:
      S_k(T) = RN32(S_{k-1} * sigmoid32(RN32(z_k / T)))   (S_0 = 1)
      ECE_k(T) from S_k(T) and the labels y_k = prefix_mask[:, k-1]
  T_k = the candidate with the smallest ECE (the first one on ties);
  S_k = S_k(T_k).

Readings (also in the design notes):
* The temperature grid and the number of bins are the caller's; bins are
  equal-width over [0, 1], bin = min(floor(S * nbins), nbins - 1) with the
  product taken exactly (S in float64).
* Since |I_b| * |acc - conf| = |sum of labels in b - sum of S in b|,
  n * ECE = sum_b |L_b - C_b|. Each S enters C_b at a resolution of 2**-40
  (nearest, ties to even), as for tau in the planner, so every sum is an
  exact integer and the argmin over T is exact and order-independent.
* Brier = mean (S - y)^2, each term at 2**-40 resolution likewise; it is
  reported for the chosen T and decides nothing.
* The sigmoid is the correctly rounded one of the planner (oracle/sigmoid.py).
* A NaN survival (only a NaN logit makes one) is binned and summed as 0; the
  stored survival stays NaN.
"""

from __future__ import annotations

import numpy as np

from .sigmoid import sigmoid32

FX = 2.0 ** 40


def _fx(v64: np.ndarray) -> np.ndarray:
    """float64 values in [0, 1] at 2**-40 resolution, nearest, ties to even."""
    return np.rint(v64 * FX).astype(np.int64)


def _nan_as_zero(S) -> np.ndarray:
    """float64 survivals; a NaN (only a NaN logit makes one) counts as 0."""
    S64 = np.asarray(S, dtype=np.float32).astype(np.float64)
    return np.where(np.isnan(S64), 0.0, S64)


def ece_terms(S: np.ndarray, y: np.ndarray, nbins: int):
    """Per-bin (count, label sum, S sum at 2**-40) and the exact n * ECE * 2**40."""
    S64 = _nan_as_zero(S)
    y = np.asarray(y).astype(np.int64)
    b = np.minimum(np.floor(S64 * nbins).astype(np.int64), nbins - 1)
    count = np.bincount(b, minlength=nbins).astype(np.int64)
    labels = np.bincount(b, weights=y, minlength=nbins).astype(np.int64)
    conf = np.zeros(nbins, dtype=np.int64)
    np.add.at(conf, b, _fx(S64))
    err = int(np.sum(np.abs(labels * (1 << 40) - conf)))
    return count, labels, conf, err


def brier_fx(S: np.ndarray, y: np.ndarray) -> int:
    """n * Brier * 2**40, each squared error at 2**-40 resolution."""
    d = _nan_as_zero(S) - np.asarray(y, dtype=np.float64)
    return int(np.sum(_fx(d * d)))  # d and d * d each rounded to float64 (IEEE)


def sts_fit(z, prefix_mask, t_grid, nbins):
    """Fit one temperature per position. Returns a dict: ``temps`` float32[gamma],
    ``t_index`` int32[gamma], ``ece`` float64[gamma], ``brier`` float64[gamma],
    ``survival`` float32[N, gamma], ``ece_fx`` int64[gamma, nT] (n * ECE *
    2**40 for every candidate)."""
    z = np.asarray(z, dtype=np.float32)
    y = np.asarray(prefix_mask).astype(np.int64)
    grid = np.asarray(t_grid, dtype=np.float32)
    N, gamma = z.shape
    nT = grid.size
    S_prev = np.ones(N, dtype=np.float32)
    temps = np.zeros(gamma, dtype=np.float32)
    idx = np.zeros(gamma, dtype=np.int32)
    ece = np.zeros(gamma)
    brier = np.zeros(gamma)
    surv = np.zeros((N, gamma), dtype=np.float32)
    ece_all = np.zeros((gamma, nT), dtype=np.int64)
    for k in range(gamma):
        best, best_err, best_S = -1, None, None
        for t in range(nT):
            with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
                x = z[:, k] / grid[t]  # float32 IEEE division
            S = (S_prev * sigmoid32(x)).astype(np.float32)  # float32 product, nearest
            err = ece_terms(S, y[:, k], nbins)[3]
            ece_all[k, t] = err
            if best_err is None or err < best_err:
                best, best_err, best_S = t, err, S
        temps[k] = grid[best]
        idx[k] = best
        ece[k] = best_err / (N * FX) if N else 0.0
        brier[k] = brier_fx(best_S, y[:, k]) / (N * FX) if N else 0.0
        surv[:, k] = best_S
        S_prev = best_S
    return {"temps": temps, "t_index": idx, "ece": ece, "brier": brier, "survival": surv,
            "ece_fx": ece_all}
