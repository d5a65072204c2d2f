"""Pins for the planner's 1D SPS cost mode and graph-tier alignment.

Fixed by the pages: the floor lookup (the nearest probe not above M, no
interpolation), the 1 ms / 1.4 ms budget comparison restated as steps per
second (3620 vs about 3014 tokens/s, so the smaller budget wins), and the
37-row example (a 64-row tier: without alignment 37 real rows and 27 of
padding; with it, real candidates fill the paid rows, but only as many as
exist, and the next tier is never entered). Also fixed by brute force over
every split with exact rationals (including a table with an SPS cliff) and
by reduction to the pinned planner: the aligned lengths are the planner's
top-b allocation at the executed budget.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.plan import clamp_lens
from conftest import golden


def test_sps_floor_lookup():
    m = [8, 16, 32, 64]
    v = np.array([100.0, 90.0, 70.0, 40.0], np.float32)
    assert oracle.sps_floor(m, v, 20) == 90.0
    assert oracle.sps_floor(m, v, 16) == 90.0
    assert oracle.sps_floor(m, v, 63) == 70.0
    assert oracle.sps_floor(m, v, 64) == 40.0
    assert oracle.sps_floor(m, v, 1000) == 40.0
    assert oracle.sps_floor(m, v, 7) == 100.0  # below the first probe


def test_sps_cost_comparison_from_pages():
    g = golden("budget_cost_example.json")
    cond = np.array(g["cond"], dtype=np.float32)
    B, gamma = cond.shape
    # probes at every total M = B + b; the two budgets of the example cost 1 ms
    # and 1.4 ms per step, every other budget is made slow
    sps_m = np.arange(B, B * (gamma + 1) + 1, dtype=np.int32)
    sps = np.full(sps_m.size, 1.0, dtype=np.float32)
    for c in g["candidates"]:
        sps[c["extra"]] = np.float32(1000.0 / c["step_ms"])
    out = oracle.plan(B, gamma, oracle.IN_COND, cond, None, 1, gamma + 1, 0.0, 0, -1,
                      0.0, None, None, cost_mode=oracle.COST_SPS1D, sps_m=sps_m, sps=sps)
    sw = out["sweep"]
    assert abs(sw[2, 1] - 3620.0) < 1e-3
    assert abs(sw[3, 1] - 3014.0) < 1.0  # the page's "about 3014"
    assert out["meta"][0] == g["chosen_extra"]
    assert out["verify_lens"].tolist() == [3, 1]


def _brute_force_sps(B, gamma, s, lmin, lmax, eps, b_lo, b_hi, sps_m, sps):
    eps32 = np.float32(eps)
    n_e = sum(1 for r in range(B) for k in range(lmin, lmax) if s[r, k - 1] >= eps32)
    lo = min(max(b_lo, 0), n_e)
    hi = n_e if b_hi < 0 else min(b_hi, n_e)
    forced = sum(Fraction(float(s[r, c])) for r in range(B) for c in range(lmin - 1))
    results = {}
    for ls in itertools.product(range(lmin, lmax + 1), repeat=B):
        if any(s[r, k - 1] < eps32 for r in range(B) for k in range(lmin, ls[r])):
            continue
        b = sum(l - lmin for l in ls)
        if not lo <= b <= hi:
            continue
        tau = B + forced + sum(Fraction(float(s[r, k - 1])) for r in range(B) for k in range(lmin, ls[r]))
        M = sum(ls)
        below = [i for i, m in enumerate(sps_m) if m <= M]  # floor lookup, written out
        S = Fraction(float(sps[below[-1] if below else 0]))
        results[ls] = (float(tau * S), b)
    best = max(v[0] for v in results.values())
    best_b = min(v[1] for v in results.values() if v[0] == best)
    winners = {ls for ls, v in results.items() if v[0] == best and v[1] == best_b}
    return best, best_b, winners


def _cliff_sps(rng, B, gamma):
    """Probes at a few totals M with falling steps/s and one sharp cliff."""
    top = B * (gamma + 1)
    pts = sorted(set(rng.integers(B, top + 1, size=4).tolist()) | {B})
    vals = 200.0 - 8.0 * np.arange(len(pts))
    cut = int(rng.integers(1, len(pts))) if len(pts) > 1 else 0
    vals[cut:] -= 120.0  # the cliff
    return np.array(pts, np.int32), vals.astype(np.float32)


@pytest.mark.parametrize("seed", range(30))
def test_sps_brute_force_over_all_splits(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 4))
    gamma = int(rng.integers(1, 5))
    c = (rng.integers(20, 65, size=(B, gamma)) / 64.0).astype(np.float32)
    if seed % 5 == 0:
        c[:] = np.float32(0.75)
    lmin = int(rng.integers(1, 3))
    lmax = int(rng.integers(lmin, gamma + 2))
    eps = float(rng.choice([0.0, 0.05, 0.2]))
    b_lo = int(rng.integers(0, 2))
    b_hi = int(rng.choice([-1, b_lo + 1, b_lo + 4]))
    sps_m, sps = _cliff_sps(rng, B, gamma)
    out = oracle.plan(B, gamma, oracle.IN_COND, c, None, lmin, lmax, eps, b_lo, b_hi, 0.0,
                      None, None, cost_mode=oracle.COST_SPS1D, sps_m=sps_m, sps=sps)
    lmin_c, lmax_c = clamp_lens(gamma, lmin, lmax)
    best, best_b, winners = _brute_force_sps(B, gamma, out["survival"], lmin_c, lmax_c, eps,
                                             b_lo, b_hi, sps_m, sps)
    assert out["meta"][2] == 0
    assert out["val"][1] == best
    assert out["meta"][0] == best_b
    assert tuple(out["verify_lens"].tolist()) in winners


def test_sps_bad_probes_fall_back():
    c = np.full((2, 3), 0.5, np.float32)
    args = (2, 3, oracle.IN_COND, c, None, 1, 4, 0.0, 0, -1, 0.0, None, None)
    for m, v in (([4, 4, 6], [3, 2, 1]), ([5, 3], [1, 1]), ([2, 4], [1.0, 0.0]),
                 ([2, 4], [1.0, np.nan])):
        out = oracle.plan(*args, cost_mode=oracle.COST_SPS1D, sps_m=np.array(m, np.int32),
                          sps=np.array(v, np.float32))
        assert out["meta"][2] == oracle.DATA_BAD_COST, (m, v)
        assert out["verify_lens"].tolist() == [4, 4]


def _align_case(n_requests, gamma, b_star_cost):
    """Requests with strictly ordered survivals and an additive table whose
    best budget is b_star_cost (every other budget costs more per token)."""
    B = n_requests
    c = np.linspace(0.97, 0.6, B * gamma, dtype=np.float32).reshape(B, gamma)
    alpha = np.zeros(B + 1, np.float32)
    theta = np.full(B * (gamma + 1) + 1, 1e6, np.float32)
    theta[B + b_star_cost] = 1.0
    return B, c, alpha, theta


def test_alignment_fills_the_paid_tier_from_pages():
    # 32 requests with a root row each, best budget 5: 37 real rows in the
    # 64-row tier; alignment adds the next 27 candidates, reaching 64 rows
    B, c, alpha, theta = _align_case(32, 2, 5)
    tiers = [32, 64, 96]
    plain = oracle.plan(B, 2, oracle.IN_COND, c, None, 1, 3, 0.0, 0, -1, 0.0, alpha, theta)
    assert plain["meta"][0] == 5 and plain["meta"][3] == 37
    out = oracle.plan(B, 2, oracle.IN_COND, c, None, 1, 3, 0.0, 0, -1, 0.0, alpha, theta,
                      align_tiers=tiers)
    assert out["meta"][0] == 5  # the argmax budget is unchanged
    assert out["meta"][3] == 64  # 27 rows of padding reclaimed
    assert int(out["verify_lens"].sum()) == 64
    assert np.array_equal(out["val"], plain["val"])


def test_alignment_cannot_force_rows():
    # eps leaves only 12 candidates: 32 + 5 chosen, at most 32 + 12 executed
    B, c, alpha, theta = _align_case(32, 2, 5)
    s, _ = oracle.survival(oracle.IN_COND, c)
    eps = float(np.sort(s[:, :2].reshape(-1))[::-1][11])
    out = oracle.plan(B, 2, oracle.IN_COND, c, None, 1, 3, eps, 0, -1, 0.0, alpha, theta,
                      align_tiers=[32, 64, 96])
    assert out["meta"][1] == 12
    assert out["meta"][3] == 32 + 12


@pytest.mark.parametrize("seed", range(10))
def test_alignment_is_the_top_b_allocation_and_keeps_the_tier(seed):
    rng = np.random.default_rng(2000 + seed)
    B, gamma = int(rng.integers(2, 12)), int(rng.integers(1, 6))
    c = (rng.integers(16, 65, size=(B, gamma)) / 64.0).astype(np.float32)
    alpha = (np.arange(B + 1) / 32.0).astype(np.float32)
    theta = np.cumsum(rng.integers(1, 9, size=B * (gamma + 1) + 1) / 64.0).astype(np.float32)
    top = B * (gamma + 1)
    tiers = sorted(set(rng.integers(B, top + 1, size=3).tolist()) | {top})
    eps = float(rng.choice([0.0, 0.1, 0.3]))
    b_hi = int(rng.choice([-1, 1, 3]))
    out = oracle.plan(B, gamma, oracle.IN_COND, c, None, 1, gamma + 1, eps, 0, b_hi, 0.0, alpha,
                      theta, align_tiers=tiers)
    ref = oracle.plan(B, gamma, oracle.IN_COND, c, None, 1, gamma + 1, eps, 0, b_hi, 0.0, alpha,
                      theta)
    b_star, n_e = int(ref["meta"][0]), int(ref["meta"][1])
    assert out["meta"][0] == b_star
    total = B + b_star
    tier = next(t for t in tiers if t >= total)
    b_exec = int(out["meta"][3]) - B
    assert b_star <= b_exec <= n_e
    assert B + b_exec <= tier
    assert b_exec == n_e or B + b_exec == tier  # filled as far as candidates and tier allow
    assert next(t for t in tiers if t >= B + b_exec) == tier  # the same tier
    # the top-b_exec allocation of the same sorted list
    forced = oracle.plan(B, gamma, oracle.IN_COND, c, None, 1, gamma + 1, eps, b_exec, b_exec,
                         0.0, alpha, theta)
    assert np.array_equal(out["verify_lens"], forced["verify_lens"])
    assert np.all(out["verify_lens"] >= ref["verify_lens"])
