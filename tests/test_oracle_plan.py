"""Pins for the planner oracle (STS -> survival -> top-b budget -> verify_lens).

What fixes each part, independently of the oracle's own code:

* the pages' printed examples (golden fixtures): the two-request allocation
  with budget 2 (verify_lens [3,1], tau 3.62), the 3620 vs ~3014 tokens/s
  teaching comparison, and the survival-by-depth table;
* the Tiny workload's full sweep, worked by hand from the tau and cost
  formulas: b* = 6, verify_lens [5,3], tau 5.3264, ratio 7.8329 per ms;
* brute force over every split (l_1..l_B) of tiny instances with exact
  rationals, including cost tables with a cliff, as the pages describe the
  scheduler's own cliff-table brute-force test;
* invariants stated in prose on the pages: survival never increases along a
  request, the top-b selection keeps each request's prefix, and each length
  lies in [L_min, L_max].
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.plan import clamp_lens
from conftest import golden
from workloads import make


def _flat_cost(B, gamma, t=1.0):
    alpha = np.zeros(B + 1, dtype=np.float32)
    theta = np.full(B * (gamma + 1) + 1, t, dtype=np.float32)
    return np.float32(0.0), alpha, theta


def test_budget_example_from_pages():
    g = golden("budget_example.json")
    cond = np.array(g["cond"], dtype=np.float32)
    B, gamma = cond.shape
    bias, alpha, theta = _flat_cost(B, gamma)
    eb = g["extra_budget"]
    out = oracle.plan(B, gamma, oracle.IN_COND, cond, None, 1, gamma + 1, 0.0, eb, eb,
                      bias, alpha, theta)
    assert out["verify_lens"].tolist() == g["verify_lens"]
    assert abs(out["val"][0] - g["tau"]) < 1e-6
    assert np.allclose(out["survival"], np.array(g["survival"]), atol=1e-7)
    assert out["meta"][0] == eb


def test_cost_comparison_from_pages():
    g = golden("budget_cost_example.json")
    cond = np.array(g["cond"], dtype=np.float32)
    B, gamma = cond.shape
    alpha = np.zeros(B + 1, dtype=np.float32)
    theta = np.full(B * (gamma + 1) + 1, 1e6, dtype=np.float32)  # other budgets: huge step time
    for c in g["candidates"]:
        theta[B + c["extra"]] = c["step_ms"]
    out = oracle.plan(B, gamma, oracle.IN_COND, cond, None, 1, gamma + 1, 0.0, 2, 3,
                      np.float32(0.0), alpha, theta)
    sw = out["sweep"]
    assert abs(sw[2, 0] - 3.62) < 1e-6 and abs(sw[3, 0] - 4.22) < 1e-6
    assert abs(sw[2, 1] * 1000 - 3620.0) < 1e-3
    assert abs(sw[3, 1] * 1000 - 3014.0) < 1.0  # the page's "about 3014"
    assert out["meta"][0] == g["chosen_extra"]
    assert out["verify_lens"].tolist() == [3, 1]


def test_survival_table_from_pages():
    g = golden("survival_table.json")
    c = np.array([g["cond"]], dtype=np.float32)
    s, bad = oracle.survival(oracle.IN_COND, c)
    assert not bad
    printed = np.array(g["printed_survival"])
    diff = np.abs(s[0].astype(np.float64) - printed)
    assert np.all(diff <= 1.5e-3)
    # five entries agree to rounding; depth 3 is the page's erratum (0.664, printed 0.665)
    assert np.sum(diff <= 5e-4) == 5 and diff[2] > 5e-4
    assert abs(float(s[0, 2]) - 0.664) < 5e-4
    assert np.all(np.diff(s[0]) <= 0)


def test_tiny_full_sweep_worked_by_hand():
    w = make(0, logits=False)
    out = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                      w.max_len, w.eps, 0, 8, w.bias, w.alpha, w.theta)
    assert out["meta"][0] == 6
    assert out["verify_lens"].tolist() == [5, 3]
    assert abs(out["val"][0] - 5.3264) < 1e-5
    assert abs(out["val"][1] - 7.8329) < 1e-4
    # capped at 2: ratios 3.571, 5.000, 6.033 per ms, so b* = 2 -> [3, 1], tau 3.62
    cap = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                      w.max_len, w.eps, 0, 2, w.bias, w.alpha, w.theta)
    assert cap["verify_lens"].tolist() == [3, 1]
    assert abs(cap["val"][0] - 3.62) < 1e-5
    assert np.allclose(cap["sweep"][:3, 1], [2 / 0.56, 2.9 / 0.58, 3.62 / 0.60], atol=1e-4)


def _brute_force(B, gamma, s, lmin, lmax, eps, b_lo, b_hi, bias, alpha, theta):
    """Exact best ratio over all splits; returns (best RN64 ratio, smallest b, set of lens)."""
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
        if not (lo <= b <= hi):
            continue
        tau = B + forced + sum(Fraction(float(s[r, k - 1])) for r in range(B) for k in range(lmin, ls[r]))
        T = Fraction(float(bias)) + Fraction(float(alpha[B])) + Fraction(float(theta[B * lmin + b]))
        results[ls] = (float(tau / T), b)
    best = max(v[0] for v in results.values())
    best_b = min(v[1] for v in results.values() if v[0] == best)
    winners = {ls for ls, v in results.items() if v[0] == best and v[1] == best_b}
    return best, best_b, winners


def _dyadic_table(rng, n, cliff):
    steps = rng.integers(1, 9, size=n).astype(np.float64) / 64.0
    if cliff:
        m0 = int(rng.integers(2, max(3, n - 1)))
        steps[m0] += float(rng.integers(4, 40)) / 8.0  # a step up in cost at one M
    return np.cumsum(steps).astype(np.float32)


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_over_all_splits(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    gamma = int(rng.integers(1, 5))
    # conditional confidences on a 1/64 grid keep every survival >= 2**-17
    c = (rng.integers(20, 65, size=(B, gamma)) / 64.0).astype(np.float32)
    if seed % 5 == 0:  # exact ties across requests and positions
        c[:] = np.float32(0.75)
    lmin = int(rng.integers(1, 3))
    lmax = int(rng.integers(lmin, gamma + 2))
    eps = float(rng.choice([0.0, 0.05, 0.2, 0.5]))
    b_lo = int(rng.integers(0, 3))
    b_hi = int(rng.choice([-1, b_lo, b_lo + 1, b_lo + 4]))
    bias = np.float32(rng.integers(0, 9) / 16.0)
    alpha = (np.arange(B + 1) / 32.0).astype(np.float32)
    theta = _dyadic_table(rng, B * (gamma + 1) + 1, cliff=(seed % 2 == 1))
    out = oracle.plan(B, gamma, oracle.IN_COND, c, None, lmin, lmax, eps, b_lo, b_hi,
                      bias, alpha, theta)
    lmin_c, lmax_c = clamp_lens(gamma, lmin, lmax)
    best, best_b, winners = _brute_force(B, gamma, out["survival"], lmin_c, lmax_c, eps,
                                         b_lo, b_hi, bias, alpha, theta)
    assert out["meta"][2] == 0
    assert out["val"][1] == best
    assert out["meta"][0] == best_b
    assert tuple(out["verify_lens"].tolist()) in winners


def _check_invariants(w, out):
    s = out["survival"]
    lmin, lmax = out["lmin"], out["lmax"]
    lens = out["verify_lens"]
    assert np.all(s[:, 1:] <= s[:, :-1])
    assert np.all((lens >= lmin) & (lens <= lmax))
    assert int(np.sum(lens - lmin)) == out["meta"][0]
    eps32 = np.float32(w.eps)
    # every selected candidate beats every unselected eligible one under the sort key
    sel, unsel = [], []
    for r in range(w.B):
        for k in range(lmin, lmax):
            if s[r, k - 1] < eps32:
                continue
            key = (-float(s[r, k - 1]), k, r)
            (sel if k < lens[r] else unsel).append(key)
    if sel and unsel:
        assert max(sel) < min(unsel)
    # tau(b) increments are the sorted survivals: non-increasing
    sw = out["sweep"][: out["meta"][1] + 1, 0]
    inc = np.diff(sw)
    assert np.all(inc >= 0) and np.all(np.diff(inc) <= 1e-12)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
@pytest.mark.parametrize("seed", [None, 11, 12])
def test_invariants_on_workloads(cfg, seed):
    w = make(cfg, seed=seed, logits=False)
    out = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                      w.max_len, w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    assert out["meta"][2] == 0
    _check_invariants(w, out)


def test_input_kinds_agree():
    w = make(1, logits=False)
    a = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, 1, 9, w.eps,
                    w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    c = oracle.sigmoid32(w.conf / w.temps[None, :])
    b = oracle.plan(w.B, w.gamma, oracle.IN_COND, c, None, 1, 9, w.eps, w.b_lo, w.b_hi,
                    w.bias, w.alpha, w.theta)
    s = oracle.plan(w.B, w.gamma, oracle.IN_SURVIVAL, a["survival"], None, 1, 9, w.eps,
                    w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    for o in (b, s):
        assert np.array_equal(o["verify_lens"], a["verify_lens"])
        assert np.array_equal(o["meta"], a["meta"])
        assert np.array_equal(o["val"], a["val"])


def test_min_len_forces_rows_and_counts_their_survival():
    c = np.array([[0.5, 0.5, 0.5], [0.9, 0.9, 0.9]], dtype=np.float32)
    bias, alpha, theta = _flat_cost(2, 3)
    out = oracle.plan(2, 3, oracle.IN_COND, c, None, 2, 4, 0.0, 0, 0, bias, alpha, theta)
    assert out["verify_lens"].tolist() == [2, 2]
    assert abs(out["val"][0] - (2 + 0.5 + 0.9)) < 1e-6


def test_eps_drops_candidates_and_max_len_caps():
    c = np.array([[0.9, 0.9, 0.01, 0.9]], dtype=np.float32)
    bias, alpha, theta = _flat_cost(1, 4)
    out = oracle.plan(1, 4, oracle.IN_COND, c, None, 1, 5, 0.05, 0, -1, bias, alpha, theta)
    assert out["meta"][1] == 2  # positions 3, 4 fall below eps (survival is a product)
    assert out["verify_lens"].tolist() == [3]
    out = oracle.plan(1, 4, oracle.IN_COND, c, None, 1, 2, 0.0, 0, -1, bias, alpha, theta)
    assert out["verify_lens"].tolist() == [2]


def test_degenerate_cases():
    bias, alpha, theta = _flat_cost(3, 2)
    c = np.full((3, 2), 0.5, dtype=np.float32)
    # min == max: no candidates, budget 0
    out = oracle.plan(3, 2, oracle.IN_COND, c, None, 2, 2, 0.0, 0, -1, bias, alpha, theta)
    assert out["meta"][1] == 0 and out["verify_lens"].tolist() == [2, 2, 2]
    # all survivals equal: ties go to earlier position, then lower request
    out = oracle.plan(3, 2, oracle.IN_COND, c, None, 1, 3, 0.0, 2, 2, bias, alpha, theta)
    assert out["verify_lens"].tolist() == [2, 2, 1]
    # B = 0
    out = oracle.plan(0, 2, oracle.IN_COND, np.zeros((0, 2), np.float32), None, 1, 3, 0.0, 0, -1,
                      bias, alpha, theta)
    assert out["verify_lens"].size == 0 and out["meta"][0] == 0


def test_bad_data_falls_back_to_static_window():
    w = make(1, logits=False)
    theta = w.theta.copy()
    theta[w.B + 3] = -10.0  # T = bias + alpha(B) + theta < 0 at M = B + 3
    out = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, 1, 9, w.eps,
                      w.b_lo, w.b_hi, w.bias, w.alpha, theta)
    assert out["meta"][2] == oracle.DATA_BAD_COST
    assert np.all(out["verify_lens"] == 9) and out["meta"][0] == -1
    temps = w.temps.copy()
    temps[2] = -1.0
    out = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, temps, 1, 9, w.eps,
                      w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    assert out["meta"][2] == oracle.DATA_BAD_CONF and np.all(out["verify_lens"] == 9)
    bad_s = np.array([[0.5, 0.6]], dtype=np.float32)
    bias, alpha, theta = _flat_cost(1, 2)
    out = oracle.plan(1, 2, oracle.IN_SURVIVAL, bad_s, None, 1, 3, 0.0, 0, -1, bias, alpha, theta)
    assert out["meta"][2] == oracle.DATA_BAD_CONF


def test_tie_rule_prefers_earlier_position_over_lower_request():
    # request 0 reaches survival 0.5 at position 2, request 1 at position 1:
    # the earlier position wins the tie, whatever the request ids
    c = np.array([[1.0, 0.5], [0.5, 1.0]], dtype=np.float32)
    bias, alpha, theta = _flat_cost(2, 2)
    out = oracle.plan(2, 2, oracle.IN_COND, c, None, 1, 3, 0.0, 2, 2, bias, alpha, theta)
    assert out["verify_lens"].tolist() == [2, 2]


def test_equal_ratios_take_the_smaller_budget():
    # s = [0.5, 0.5]: tau(0..2) = 1, 1.5, 2; T = 2, 1.5, 2 -> ratios 0.5, 1, 1
    c = np.array([[0.5, 1.0]], dtype=np.float32)
    alpha = np.zeros(2, dtype=np.float32)
    theta = np.array([9.0, 2.0, 1.5, 2.0], dtype=np.float32)
    out = oracle.plan(1, 2, oracle.IN_COND, c, None, 1, 3, 0.0, 0, -1, np.float32(0), alpha, theta)
    assert out["sweep"][1, 1] == out["sweep"][2, 1] == 1.0
    assert out["meta"][0] == 1 and out["verify_lens"].tolist() == [2]


def test_eps_cutoff_keeps_values_equal_to_eps():
    c = np.array([[0.5, 0.5]], dtype=np.float32)  # survivals 0.5, 0.25
    bias, alpha, theta = _flat_cost(1, 2)
    out = oracle.plan(1, 2, oracle.IN_COND, c, None, 1, 3, 0.25, 0, -1, bias, alpha, theta)
    assert out["meta"][1] == 2
    out = oracle.plan(1, 2, oracle.IN_COND, c, None, 1, 3, 0.2500001, 0, -1, bias, alpha, theta)
    assert out["meta"][1] == 1


def test_negative_zero_survival_ranks_with_zero():
    # survivals (0.5, -0), (0.9, 0.72): the order is by value, so -0 comes last
    # and a budget of 2 takes request 1's two positions
    c = np.array([[0.5, -0.0], [0.9, 0.8]], dtype=np.float32)
    bias, alpha, theta = _flat_cost(2, 2)
    out = oracle.plan(2, 2, oracle.IN_COND, c, None, 1, 3, 0.0, 2, 2, bias, alpha, theta)
    assert out["verify_lens"].tolist() == [1, 3]
    assert out["meta"][1] == 4  # -0 >= eps = 0: a candidate
    # -0 and +0 give the same plan (only the survival's sign bit differs)
    cp = np.abs(c)
    for lo, hi in ((0, -1), (3, 4), (4, 4)):
        a = oracle.plan(2, 2, oracle.IN_COND, c, None, 1, 3, 0.0, lo, hi, bias, alpha, theta)
        b = oracle.plan(2, 2, oracle.IN_COND, cp, None, 1, 3, 0.0, lo, hi, bias, alpha, theta)
        assert a["verify_lens"].tolist() == b["verify_lens"].tolist()
        assert np.array_equal(a["meta"], b["meta"])
        assert np.array_equal(a["sweep"], b["sweep"], equal_nan=True)
