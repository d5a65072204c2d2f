"""Pins for the fixed-resolution (integer-weight) form of the sampling accept,
the white-box check of the kernels' arithmetic (``oracle.sampling_fixed``).
The definition itself is the float64 ``oracle.sampling``, pinned in
``test_oracle_sampling.py``; the last tests here tie the two together: the
per-token error of the fixed resolution stays inside the bound the float64
validator's band is built from, and the fixed form's decisions pass that
validator.

Fixed by:
* the exp2 table against an independent 80-bit long-double evaluation, and
  K against a 50-digit decimal 2^16 / ln 2;
* the fixed-resolution probabilities against the float64 softmax (closed
  form), the value 2^31 at the maximum, table entries hit exactly,
  monotonicity and the power-of-two scaling invariance of x / T;
* the theorem of speculative sampling: one chain step outputs a token
  distributed exactly as p (to the 2^-24 resolution of the random words),
  whatever q is, and its acceptance rate is sum min(p, q) = 1 - TV, the
  pages' identity; both computed by exhaustive counting over all 2^24
  values of each random word, with the oracle's own decision functions;
* closed cases: p == q always accepts, disjoint one-hot rows always reject
  and resample the target token, a draft outside the vocabulary is rejected;
* the greedy path (temperature 0) equal to the greedy accept oracle;
* compaction invariance: compact accept with length l agrees with the
  full-width (static) accept under the same random words wherever the
  static chain stops before l - 1 ([CSSD], compact vs static).
"""

import numpy as np
import pytest

import oracle
from oracle import sampling as F64
from oracle import sampling_fixed as S


def test_exp_table_against_long_double():
    Bt = S.exp_table()
    ld = np.longdouble
    assert np.finfo(ld).eps < 1e-18  # 80-bit extended on this host
    assert len(Bt) == S.B_LEN == 257
    for i, v in enumerate(Bt):
        ref = ld(2) ** (31 - ld(i) / 256)
        assert abs(ld(v) - ref) <= 0.5 + ref * 1e-17, (i, v, ref)
    assert Bt[0] == 2**31 and Bt[256] == 2**30
    # K is the float32 nearest to 2^16 log2(e)
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    k = Decimal(65536) / Decimal(2).ln()
    below = np.nextafter(S.K_LOG2E_16, np.float32(0))
    above = np.nextafter(S.K_LOG2E_16, np.float32(1e9))
    d0 = abs(Decimal(float(S.K_LOG2E_16)) - k)
    assert d0 < abs(Decimal(float(below)) - k) and d0 < abs(Decimal(float(above)) - k)


@pytest.mark.parametrize("T", [0.05, 0.6, 1.0, 1.7, 8.0])
def test_weights_match_softmax(T):
    rng = np.random.default_rng(int(T * 100))
    x = rng.normal(0.0, 3.0, 5000).astype(np.float32)
    W = S.weights(x, T)
    assert W.max() == 2**31 and W[np.argmax(x)] == 2**31
    p = W.astype(np.float64) / float(W.sum())
    y = (x.astype(np.float64) - x.max()) / np.float64(np.float32(T))
    q = np.exp(y) / np.exp(y).sum()
    big = q > 1e-3 * q.max()  # W above 2^21: the 2^-31 grid is below 5e-7 relative
    assert np.max(np.abs(p - q)[big] / q[big]) < 1.5e-5
    assert 0.5 * np.abs(p - q).sum() < 1e-5
    # monotone in the logit (up to one unit of the interpolation's rounding)
    order = np.argsort(x, kind="stable")
    Wo = W[order]
    assert np.all(np.diff(Wo) >= -1)
    assert np.all(np.diff(Wo)[Wo[:-1] > 2**16] >= 0)


def test_weights_scaling_invariance_and_special_values():
    rng = np.random.default_rng(2)
    x = rng.normal(0.0, 4.0, 3000).astype(np.float32)
    for T in (0.3, 1.0, 2.5):
        assert np.array_equal(S.weights(x, T), S.weights(x * 4, T * 4))
        assert np.array_equal(S.weights(x, T), S.weights(x / 8, T / 8))
    # -inf has weight 0; a logit 30 below the max at T = 1 is below 2^-32
    z = np.array([0.0, -np.inf, -30.0, -1.0, -22.0], np.float32)
    W = S.weights(z, 1.0)
    assert W[0] == 2**31 and W[1] == 0 and W[2] == 0
    assert abs(int(W[3]) - 2**31 * np.exp(-1.0)) < 2**31 * 1e-5
    assert abs(int(W[4]) - 2**31 * np.exp(-22.0)) <= 1
    # j = 256 i lands on table entries, shifted by the octave: W = round(B[i % 256] / 2^n)
    Bt = S.exp_table()
    for i in (1, 7, 100, 4000):
        x = np.array([0.0, -np.float32(i * 256) / np.float32(S.K_LOG2E_16)], np.float32)
        u = (x[0] - x[1]) * S.K_LOG2E_16
        if np.rint(u) == i * 256:
            n = i >> 8
            assert S.weights(x, 1.0)[1] == (Bt[i & 255] + ((1 << n) >> 1)) >> n


def _count_accept(Wp_d, Zp, Wq_d, Zq):
    """#u in [0, 2^24) accepted: the test is monotone in u, so bisect."""
    lo, hi = 0, 1 << 24  # accepts(lo - 1) true, accepts(hi) false
    if not S.accepts(Wp_d, Zp, Wq_d, Zq, 0):
        return 0
    if S.accepts(Wp_d, Zp, Wq_d, Zq, ((1 << 24) - 1) << 8):
        return 1 << 24
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if S.accepts(Wp_d, Zp, Wq_d, Zq, mid << 8):
            lo = mid
        else:
            hi = mid
    return hi


def _draw_counts(w):
    """#v in [0, 2^24) drawing each index: draw is monotone in v, so bisect
    for the first v of each index."""
    n = len(w)
    first = []
    for i in range(n + 1):
        lo, hi = 0, 1 << 24
        while lo < hi:  # first v with draw(v) >= i
            mid = (lo + hi) // 2
            if S.draw(w, mid << 8) >= i:
                hi = mid
            else:
                lo = mid + 1
        first.append(lo)
    first[n] = 1 << 24
    return np.diff(np.array(first, dtype=np.int64))


@pytest.mark.parametrize("seed", range(6))
def test_one_chain_step_outputs_the_target_distribution(seed):
    rng = np.random.default_rng(100 + seed)
    V = 6
    p_row = rng.normal(0, 2, V).astype(np.float32)
    q_row = rng.normal(0, 2, V).astype(np.float32)
    if seed == 5:
        q_row[2] = -np.inf  # the draft never proposes token 2
    T = [1.0, 0.5, 2.0, 1.0, 0.8, 1.0][seed]
    Wp, Wq = S.weights(p_row, T), S.weights(q_row, T)
    Zp, Zq = int(Wp.sum()), int(Wq.sum())
    p = np.array([int(v) for v in Wp], dtype=object)
    R = S.residual(Wp, Zp, Wq, Zq)
    rho = _draw_counts(R if int(np.sum(R)) else Wp)
    out = np.zeros(V)
    acc_rate = 0.0
    for d in range(V):
        qd = int(Wq[d]) / Zq
        a = _count_accept(int(Wp[d]), Zp, int(Wq[d]), Zq) / 2**24
        acc_rate += qd * a
        out[d] += qd * a
        out += qd * (1 - a) * rho / 2**24
    target = np.array([float(v) for v in p]) / Zp
    assert np.max(np.abs(out - target)) < 2 * 2.0**-24, (out, target)
    ptrue, qtrue = Wp.astype(np.float64) / Zp, Wq.astype(np.float64) / Zq
    assert abs(acc_rate - np.minimum(ptrue, qtrue).sum()) < 2 * 2.0**-24
    assert abs(acc_rate - (1 - 0.5 * np.abs(ptrue - qtrue).sum())) < 2 * 2.0**-24


def _batch(rng, B, gamma, V, lens, dtype="f32"):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tgt = rng.normal(0, 2, (int(cu[-1]) + 3, V)).astype(np.float32)
    drf = rng.normal(0, 2, (B * gamma, V)).astype(np.float32)
    drafts = rng.integers(0, V, (B, gamma)).astype(np.int32)
    ra = rng.integers(0, 2**32, (B, gamma), dtype=np.uint64).astype(np.uint32)
    rs = rng.integers(0, 2**32, (B, gamma + 1), dtype=np.uint64).astype(np.uint32)
    return cu, tgt, drf, drafts, ra, rs


def test_identical_rows_always_accept_and_disjoint_rows_always_reject():
    rng = np.random.default_rng(5)
    B, gamma, V = 6, 4, 50
    lens = np.array([5, 3, 1, 5, 2, 4])
    cu, tgt, drf, drafts, ra, rs = _batch(rng, B, gamma, V, lens)
    for r in range(B):
        for k in range(1, lens[r]):
            drf[r * gamma + k - 1] = tgt[cu[r] + k - 1]
    res = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, np.ones(B), ra, rs)
    assert res["num_correct"].tolist() == (lens - 1).tolist()
    # disjoint one-hots: q proposes token 3, p puts all mass on token 7
    tgt[:] = -np.inf
    tgt[:, 7] = 0.0
    drf[:] = -np.inf
    drf[:, 3] = 0.0
    drafts[:] = 3
    res = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, np.ones(B), ra, rs)
    expect_bonus = [7 if l > 1 else 7 for l in lens]
    assert res["num_correct"].tolist() == [0] * B and res["bonus"].tolist() == expect_bonus
    assert res["status"] == 0
    # a draft outside the vocabulary is rejected even when p == q
    drf[:] = tgt[0]
    drafts[:] = V
    res = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, np.ones(B), ra, rs)
    assert res["num_correct"].tolist() == [0] * B and res["bonus"].tolist() == [7] * B


def test_greedy_requests_follow_the_greedy_oracle():
    rng = np.random.default_rng(9)
    B, gamma, V = 9, 5, 40
    lens = rng.integers(1, gamma + 2, B)
    cu, tgt, drf, drafts, ra, rs = _batch(rng, B, gamma, V, lens)
    am = oracle.row_argmax(tgt)
    for r in range(B):  # make some drafts match
        for k in range(1, lens[r]):
            if rng.random() < 0.7:
                drafts[r, k - 1] = am[cu[r] + k - 1]
    tgt[1, 4] = np.nan
    got = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, np.zeros(B), ra, rs,
                            prefix_lens=np.arange(B))
    ref = oracle.accept(B, gamma, tgt, "f32", cu, drafts, prefix_lens=np.arange(B))
    for k in ("num_correct", "bonus", "commit", "new_seq", "out_tokens"):
        assert np.array_equal(got[k], ref[k]), k


@pytest.mark.parametrize("seed", range(4))
def test_compact_agrees_with_static_under_the_same_random_words(seed):
    rng = np.random.default_rng(200 + seed)
    B, gamma, V = 12, 6, 30
    full = np.full(B, gamma + 1)
    cu_s, tgt_s, drf, drafts, ra, rs = _batch(rng, B, gamma, V, full)
    # make acceptance likely: q close to p
    for r in range(B):
        for k in range(1, gamma + 1):
            drf[r * gamma + k - 1] = tgt_s[cu_s[r] + k - 1] + rng.normal(0, 0.3, V).astype(np.float32)
    temps = rng.choice([0.7, 1.0, 1.3], B).astype(np.float32)
    static = S.accept_sampling(B, gamma, tgt_s, drf, "f32", cu_s, drafts, temps, ra, rs)
    lens = rng.integers(1, gamma + 2, B)
    cu_c = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tgt_c = np.concatenate([tgt_s[cu_s[r]:cu_s[r] + lens[r]] for r in range(B)])
    comp = S.accept_sampling(B, gamma, tgt_c, drf, "f32", cu_c, drafts, temps, ra, rs)
    assert np.array_equal(comp["num_correct"], np.minimum(static["num_correct"], lens - 1))
    stops = static["num_correct"] < lens - 1
    assert np.array_equal(comp["bonus"][stops], static["bonus"][stops])
    for r in np.flatnonzero(~stops):  # capped: the bonus is drawn from p of row l - 1
        W = S.weights(tgt_c[cu_c[r] + lens[r] - 1], temps[r])
        assert comp["bonus"][r] == S.draw(W, rs[r, lens[r] - 1])
    assert stops.any() and (~stops).any()


def test_bad_data_falls_back():
    rng = np.random.default_rng(11)
    B, gamma, V = 5, 3, 20
    lens = np.array([4, 2, 3, 1, 4])
    cu, tgt, drf, drafts, ra, rs = _batch(rng, B, gamma, V, lens)
    temps = np.array([1.0, -1.0, 1.0, np.nan, 0.0], np.float32)
    # a scale K / T that overflows float32 is out of domain too; just above
    # it, the row's maximum keeps the full weight
    tiny = np.float32(1e-34)
    assert not np.isfinite(S.temp_scale(tiny)) and np.isfinite(S.temp_scale(np.float32(3e-34)))
    assert S.weights(np.array([0.0, -1e-30], np.float32), np.float32(3e-34))[0] == 2**31
    tgt[cu[2] + 1, 3] = np.inf  # request 2's second row
    tgt[cu[4], 5] = np.nan  # greedy request: NaN is an ordinary (largest) value
    res = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, temps, ra, rs,
                            prefix_lens=np.full(B, 10))
    assert res["status"] == S.DATA_BAD_LOGITS | oracle.DATA_BAD_CONF
    t2 = temps.copy()
    t2[1] = tiny
    res2 = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, t2, ra, rs)
    assert res2["status"] == res["status"] and res2["bonus"][1] == -1
    for r in (1, 2, 3):
        assert res["num_correct"][r] == 0 and res["bonus"][r] == -1 and res["commit"][r] == 0
        assert res["new_seq"][r] == 10 and (res["out_tokens"][r] == -1).all()
    assert res["bonus"][4] == 5 and res["commit"][0] >= 1
    bad = cu.copy()
    bad[2] = bad[1]  # request 1 gets no rows
    res = S.accept_sampling(B, gamma, tgt, drf, "f32", bad, drafts, np.ones(B), ra, rs)
    assert res["status"] & oracle.DATA_BAD_LENS and res["bonus"][1] == -1


def test_bf16_rows_widen_exactly():
    rng = np.random.default_rng(12)
    B, gamma, V = 4, 3, 24
    lens = np.array([4, 4, 2, 3])
    cu, tgt, drf, drafts, ra, rs = _batch(rng, B, gamma, V, lens)
    tb = (tgt.view(np.uint32) >> 16).astype(np.uint16)
    db = (drf.view(np.uint32) >> 16).astype(np.uint16)
    a = S.accept_sampling(B, gamma, tb, db, "bf16", cu, drafts, np.ones(B), ra, rs)
    tw = (tb.astype(np.uint32) << 16).view(np.float32)
    dw = (db.astype(np.uint32) << 16).view(np.float32)
    b = S.accept_sampling(B, gamma, tw, dw, "f32", cu, drafts, np.ones(B), ra, rs)
    for k in ("num_correct", "bonus", "out_tokens"):
        assert np.array_equal(a[k], b[k])


def test_zero_probability_is_never_drawn_or_accepted():
    # counts over all 2^24 values of the word are exactly the integer shares
    w = np.array([0, 3, 0, 5, 0], dtype=object)
    counts = _draw_counts(w)
    assert counts[0] == 0 and counts[2] == 0 and counts[4] == 0
    assert counts.sum() == 2**24 and abs(counts[1] - 3 * 2**24 / 8) <= 1
    assert S.draw(w, 0) == 1 and S.draw(w, 0xFFFFFFFF) == 3
    # min(1, p/q) is 0 when p(d) = 0, whatever q(d) is
    Z = 5 * 2**31
    assert _count_accept(0, Z, 2**31, Z) == 0
    assert _count_accept(0, Z, 0, Z) == 0
    # and 1 when p(d) >= q(d) > 0
    assert _count_accept(2**31, Z, 2**31, Z) == 2**24
    assert _count_accept(2**30, Z, 2**31, Z) == 2**23


def test_each_output_column_draws_with_its_own_word():
    # one request, gamma = 3, length 4: draft 1 is always rejected (disjoint
    # rows), and the residual is p = uniform over tokens 5 and 9
    B, gamma, V = 1, 3, 12
    tgt = np.full((4, V), -np.inf, np.float32)
    tgt[:, [5, 9]] = 0.0
    drf = np.full((3, V), -np.inf, np.float32)
    drf[:, 1] = 0.0
    drafts = np.array([[1, 1, 1]], np.int32)
    cu = np.array([0, 4], np.int32)
    ra = np.zeros((1, 3), np.uint32)
    lo, hi = np.uint32(0), np.uint32(0xFFFFFFFF)
    for col0, expect in ((lo, 5), (hi, 9)):
        rs = np.array([[col0, hi - col0, hi - col0, hi - col0]], np.uint32)
        res = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, np.ones(1), ra, rs)
        assert res["num_correct"][0] == 0 and res["bonus"][0] == expect
    # all accepted (q == p, drafts in the support): column 3 draws from row 3
    drf[:] = tgt[0]
    drafts[:] = 9
    for col3, expect in ((lo, 5), (hi, 9)):
        rs = np.array([[hi - col3] * 3 + [col3]], np.uint32)
        res = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, np.ones(1), ra, rs)
        assert res["num_correct"][0] == 3 and res["bonus"][0] == expect
        assert res["out_tokens"][0].tolist() == [9, 9, 9, expect]


@pytest.mark.parametrize("T", [0.7, 1.0, 2.0])
def test_weights_are_unbiased(T):
    # nearest rounding of j leaves no systematic error: the mean signed
    # relative error of W against 2^31 exp((x - m) / T) is about 0, while a
    # floor (or any one-sided rounding) biases it by about 2^-17 ln 2 = 5e-6
    rng = np.random.default_rng(31)
    x = (rng.uniform(-22.0, 0.0, 200000) * T).astype(np.float32)
    x[0] = 0.0
    W = S.weights(x, T)
    ref = 2.0**31 * np.exp(x.astype(np.float64) / np.float64(np.float32(T)))
    big = W > 2**20
    rel = W[big] / ref[big] - 1.0
    assert abs(rel.mean()) < 1e-6, rel.mean()
    assert np.max(np.abs(rel)) < 1.2e-5
    # small weights: the interpolation rounds to nearest too (mean error in
    # units of 2^-31 about 0, not the +1/2 of a truncating interpolation)
    small = (W > 2**8) & (W < 2**14)
    assert small.sum() > 5000
    err = W[small] - ref[small]
    assert abs(err.mean()) < 0.1, err.mean()


# ---- the fixed resolution against the float64 definition

@pytest.mark.parametrize("V,T,sigma,seed", [
    (5000, 1.0, 3.0, 1), (129280, 0.7, 3.0, 2), (151936, 1.4, 3.0, 3), (32000, 0.05, 2.0, 4),
    (20000, 8.0, 4.0, 5), (4099, 0.3, 1.0, 6)])
def test_per_token_error_inside_the_validators_bound(V, T, sigma, seed):
    """|W_i / sum W - p_i| <= eps_p p_i + eta_p for every token, with (eps_p,
    eta_p) = F64.prob_error_bound(V): the band the float64 validator allows
    really covers this resolution (rows as the workloads draw them: normal,
    clipped, a planted maximum, bfloat16-rounded)."""
    rng = np.random.default_rng(seed)
    x = np.clip(rng.normal(0, sigma, V), -5 * sigma, 5 * sigma).astype(np.float32)
    x[rng.integers(V)] = 5 * sigma + 1
    x = ((x.view(np.uint32) + np.uint32(0x8000)) & np.uint32(0xFFFF0000)).view(np.float32)
    x[rng.integers(V, size=50)] = -np.inf
    W = S.weights(x, np.float32(T))
    p_int = W.astype(np.float64) / float(int(W.astype(object).sum()))
    p = F64.softmax64(x, T)
    eps_p, eta_p = F64.prob_error_bound(V)
    err = np.abs(p_int - p)
    assert np.all(err <= eps_p * p + eta_p), np.max(err - eps_p * p - eta_p)
    # the bound is not vacuous: the largest relative error on large tokens
    # uses a fair part of eps_w
    big = p > 1e-3 * p.max()
    if big.sum() > 100:
        assert np.max(err[big] / p[big]) > 0.05 * F64.EPS_W


def test_weight_error_inside_eps_w():
    """Each unnormalised weight: |W - W*| <= eps_w W* + 1/2 + 1e-5 with W* =
    2^31 exp((x - m) / T), over the whole range of u up to the cut-off and
    past it (W = 0 there, W* below 1/2)."""
    rng = np.random.default_rng(77)
    for T in (0.05, 0.37, 1.0, 2.9):
        x = (-rng.uniform(0, 24.0, 300000) * T).astype(np.float32)
        x[0] = 0.0
        W = S.weights(x, np.float32(T)).astype(np.float64)
        Ws = 2.0**31 * np.exp(x.astype(np.float64) / np.float64(np.float32(T)))
        assert np.all(np.abs(W - Ws) <= F64.EPS_W * Ws + 0.5 + 1e-5)


@pytest.mark.parametrize("seed", range(5))
def test_fixed_form_passes_the_float64_validator(seed):
    """The fixed-resolution chain's outputs satisfy the float64 definition
    everywhere outside the band (on the CPU, no GPU involved)."""
    rng = np.random.default_rng(300 + seed)
    B, gamma, V = 24, 6, [700, 3001, 12000, 4096, 999][seed]
    lens = rng.integers(1, gamma + 2, B)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tgt = rng.normal(0, 2.5, (int(cu[-1]), V)).astype(np.float32)
    drf = np.empty((B * gamma, V), np.float32)
    for r in range(B):
        for k in range(gamma):
            src = tgt[cu[r] + k] if k < lens[r] else rng.normal(0, 2.5, V)
            drf[r * gamma + k] = src + rng.normal(0, [0.05, 0.3, 1.0][r % 3], V)
    drafts = np.argmax(drf, axis=1).reshape(B, gamma).astype(np.int32)
    drafts[rng.random((B, gamma)) < 0.3] = rng.integers(0, V)
    temps = rng.uniform(0.4, 1.6, B).astype(np.float32)
    temps[rng.random(B) < 0.15] = 0.0
    ra = rng.integers(0, 2**32, (B, gamma), dtype=np.uint64).astype(np.uint32)
    rs = rng.integers(0, 2**32, (B, gamma + 1), dtype=np.uint64).astype(np.uint32)
    prefix = rng.integers(5, 500, B)
    got = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, temps, ra, rs,
                            prefix_lens=prefix)
    rep = F64.validate(B, gamma, tgt, drf, "f32", cu, drafts, temps, ra, rs, got,
                       prefix_lens=prefix)
    assert rep["failures"] == [], rep["failures"][:3]
    st = rep["stats"]
    assert st["accept_tests"] > B and st["draws_residual"] > 0 and st["draws_p"] > 0
    # the two definitions differ only inside the band, which is rare
    assert st["accept_band"] <= max(2, st["accept_tests"] // 50)
    ref = F64.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, temps, ra, rs,
                              prefix_lens=prefix)
    differ = int(np.sum(ref["num_correct"] != got["num_correct"]) +
                 np.sum((ref["num_correct"] == got["num_correct"]) & (ref["bonus"] != got["bonus"])))
    assert differ <= st["accept_band_flips"] + st["draws_p_flips"] + st["draws_residual_flips"]
