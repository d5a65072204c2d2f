"""Planner oracle: STS confidence -> survival -> top-b budget -> verify_lens.

Test infrastructure only (see ``oracle/__init__.py``).

What it computes, step by step, in the pages' order:

1. Calibrated confidence ``c[r,k] = sigmoid(z[r,k] / T[k])`` for draft
   positions k = 1..gamma ([Budget] §二, runtime STS formula).
2. Prefix survival ``s[r,k] = c[r,1] * ... * c[r,k]`` ([Budget] §一, the
   cumulative product per request; [CSSD], the prefix-event table). fp32, left
   to right.
3. All candidate positions sorted by survival, descending. Equal values go
   to the earlier position first, then the lower request id ([Budget] §一,
   the tie rule that keeps the prefix structure).
4. ``tau(b) = B + sum of the b largest survivals`` ([Budget] §一, the tau
   formula and the ``num_requests + cat([0], cumsum)`` form).
5. ``budget = argmax_b tau(b) / T(B, B + b)`` with the additive cost
   ``T = bias + alpha(B) + theta(M)`` ([Budget] §一 and §四; [CSSD], the
   cost model with ``M = bs + K``).
6. ``verify_lens``: each request keeps its root row plus the candidates of
   its own that fall in the top ``budget`` ([Budget] §一: the
   ScheduleVerifyLensTopk allocation, with min/max_verify_len and
   survival_eps).

Two variants ([Budget] §一 and §四, §五):

* 1D SPS cost mode: ``budget = argmax_b tau(b) * SPS(M)``, SPS read from a
  table of probe points by floor lookup (the nearest probe at or below M,
  no interpolation, so a cliff in the table is kept as it is).
* Graph-tier alignment (paid-padding reclamation): once the budget is
  chosen, the executed budget is extended with the next candidates in the
  same order until the packed total reaches the graph tier that the chosen
  budget already pays for; it never crosses into the next tier and never
  adds rows that are not candidates.

Readings where the pages leave a step open (each also listed in the design
notes):

* Positions ``k < L_min`` (``L_min = clamp(min_verify_len, 1, gamma+1)``) are
  always verified; positions ``k >= L_max`` never are; a position
  ``L_min <= k < L_max`` is a candidate only if ``s >= survival_eps``. The
  constraints shape the candidate list and the budget sweep runs over that
  list, so the allocation is exactly its top ``budget`` entries.
* ``M = B * L_min + b`` indexes the dense ``theta`` table: the total verify
  rows including the root rows.
* tau is an exact sum. Each survival is taken at a resolution of 2**-40
  (round to nearest, ties to even), which is exact for every survival
  >= 2**-17. Any summation order then gives the same bits. The ratio is
  the correctly rounded fp64 quotient of that exact tau by
  ``T = (bias + alpha[B]) + theta[M]`` accumulated in fp64 left to right.
* The budget range is ``[budget_lo, budget_hi]`` clipped to the number of
  candidates (``budget_hi < 0`` means no upper limit). Equal ratios go to the
  smaller budget.
* 1D mode: a total M below the first probe takes the first probe's SPS.
  The objective is the correctly rounded fp64 product ``tau * SPS``.
  Probes that are not strictly ascending, or an SPS that is not positive and
  finite at a considered budget, set DATA_BAD_COST.
* Alignment: the tier is the smallest listed tier that holds the chosen
  total ``B * L_min + b*``; the executed budget is
  ``min(b* + tier - total, #candidates)``. It ignores ``budget_hi`` (the
  cap bounds the argmax; the fill deliberately goes past it to use rows
  that are paid for). ``meta[0]`` stays the argmax budget and ``meta[3]``
  becomes the executed total.
* Bad data is detected, not trapped. A non-positive or non-finite ``T`` at a
  considered budget sets DATA_BAD_COST. Confidence outside [0, 1], a NaN, or
  a non-positive/non-finite temperature sets DATA_BAD_CONF. So does a given
  survival that is not non-increasing. In either case every request gets
  ``L_max`` rows (the static window), ``b* = -1``, and the float results are
  NaN.
"""

from __future__ import annotations

import numpy as np

from .sigmoid import sigmoid32

IN_CONF_LOGITS = 0
IN_COND = 1
IN_SURVIVAL = 2

DATA_BAD_COST = 1
DATA_BAD_CONF = 2

COST_ADDITIVE = 0
COST_SPS1D = 1

FX_SHIFT = 40  # tau resolution: 2**-40


def survival(kind: int, conf, temps=None):
    """Survival ``s[B, gamma]`` (float32) and a bad-data flag."""
    conf = np.asarray(conf, dtype=np.float32)
    B, g = conf.shape
    if kind == IN_SURVIVAL:
        s = conf.copy()
        ok = bool(np.all((s >= 0) & (s <= 1)))
        if ok and g > 1:
            ok = bool(np.all(s[:, 1:] <= s[:, :-1]))
        return s, not ok
    bad = False
    if kind == IN_CONF_LOGITS:
        T = np.asarray(temps, dtype=np.float32)
        bad = not bool(np.all(np.isfinite(T) & (T > 0)))
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            x = conf / T[None, :]  # float32 IEEE division
        c = sigmoid32(x)
    elif kind == IN_COND:
        c = conf
    else:
        raise ValueError(f"unknown input kind {kind}")
    bad = bad or not bool(np.all((c >= 0) & (c <= 1)))
    s = np.empty_like(c)
    if g:
        s[:, 0] = c[:, 0]
    for k in range(1, g):
        s[:, k] = s[:, k - 1] * c[:, k]  # float32 * float32 -> float32, round to nearest
    return s, bad


def _fx(v) -> int:
    """Survival value at the 2**-40 resolution used for tau (nearest, ties to even)."""
    return int(np.rint(np.float64(v) * 2.0 ** FX_SHIFT))


def clamp_lens(gamma: int, min_len: int, max_len: int):
    lmin = min(max(int(min_len), 1), gamma + 1)
    lmax = min(max(int(max_len), lmin), gamma + 1)
    return lmin, lmax


def sps_floor(sps_m, sps, M):
    """SPS of the nearest probe at or below M; the first probe when M is below all."""
    i = 0
    for j in range(len(sps_m)):
        if int(sps_m[j]) <= M:
            i = j
    return np.float32(sps[i])


def plan(B, gamma, kind, conf, temps, min_len, max_len, eps, budget_lo, budget_hi,
         bias, alpha, theta, cost_mode=COST_ADDITIVE, sps_m=None, sps=None, align_tiers=None):
    """Run the planner; returns a dict with the same outputs as ``dspark_plan``.

    Keys: ``verify_lens`` int32[B]; ``meta`` int32[4] = (b*, number of
    candidates, status, executed total B*L_min + b_exec); ``val`` float64[2]
    = (tau(b*), objective(b*)); ``survival`` float32[B, gamma]; ``sweep``
    float64[B*gamma+1, 2] = (tau(b), objective(b)) for b = 0..#candidates, NaN
    beyond. The objective is tau / T (additive) or tau * SPS (1D); b_exec is
    b* unless ``align_tiers`` is given."""
    B, gamma = int(B), int(gamma)
    if budget_hi >= 0 and budget_lo > budget_hi:
        raise ValueError("budget_lo > budget_hi")
    s, bad_conf = survival(kind, conf, temps)
    assert s.shape == (B, gamma)
    lmin, lmax = clamp_lens(gamma, min_len, max_len)
    eps32 = np.float32(eps)
    status = DATA_BAD_CONF if bad_conf else 0

    sweep = np.full((B * gamma + 1, 2), np.nan)
    if status == 0:
        # forced positions k = 1..L_min-1 are verified for every request
        forced = sum(_fx(s[r, c]) for r in range(B) for c in range(lmin - 1))
        # candidates: positions k = L_min..L_max-1 with s >= eps, as (s, k, r)
        cands = [(s[r, k - 1], k, r)
                 for k in range(lmin, lmax) for r in range(B)
                 if s[r, k - 1] >= eps32]
        cands.sort(key=lambda t: (-float(t[0]), t[1], t[2]))
        n_e = len(cands)
        lo = min(max(int(budget_lo), 0), n_e)
        hi = n_e if budget_hi < 0 else min(int(budget_hi), n_e)

        if cost_mode == COST_SPS1D:
            probes = [int(m) for m in sps_m]
            if not probes or any(b <= a for a, b in zip(probes, probes[1:])):
                status |= DATA_BAD_COST
        else:
            t_fixed = np.float64(bias) + np.float64(alpha[B])
        tau_fx = B * 2 ** FX_SHIFT + forced
        best_b, best_ratio = -1, None
        for b in range(n_e + 1):
            if status:
                break
            if b > 0:
                tau_fx += _fx(cands[b - 1][0])
            tau = tau_fx / 2 ** FX_SHIFT  # exact: below 2**53
            M = B * lmin + b
            if cost_mode == COST_SPS1D:
                S = np.float64(sps_floor(sps_m, sps, M))
                ratio = float(np.float64(tau) * S)
                cost_ok = bool(np.isfinite(S) and S > 0)
            else:
                T = t_fixed + np.float64(theta[M])
                ratio = float(np.float64(tau) / T)
                cost_ok = bool(np.isfinite(T) and T > 0)
            sweep[b] = (tau, ratio)
            if lo <= b <= hi:
                if not cost_ok:
                    status |= DATA_BAD_COST
                elif best_ratio is None or ratio > best_ratio:
                    best_b, best_ratio = b, ratio

    if status != 0:
        lens = np.full(B, lmax, dtype=np.int32)
        meta = np.array([-1, -1, status, B * lmax], dtype=np.int32)
        val = np.array([np.nan, np.nan])
        sweep[:] = np.nan
    else:
        b_exec = best_b
        if align_tiers is not None:
            total = B * lmin + best_b
            tier = next(int(t) for t in align_tiers if int(t) >= total)
            b_exec = min(best_b + tier - total, n_e)
        lens = np.full(B, lmin, dtype=np.int32)
        for _, _, r in cands[:b_exec]:
            lens[r] += 1
        meta = np.array([best_b, n_e, 0, B * lmin + b_exec], dtype=np.int32)
        val = sweep[best_b].copy()
    return {"verify_lens": lens, "meta": meta, "val": val, "survival": s, "sweep": sweep,
            "lmin": lmin, "lmax": lmax}
