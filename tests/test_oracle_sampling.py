"""Pins for the float64 chain speculative-sampling accept oracle
(``oracle.sampling``), the definition the GPU results are checked against.

Fixed by:
* the softmax against closed forms: a uniform row gives 1/V, the pair
  [0, -T ln 3] gives [3/4, 1/4], ratios p_i / p_j = exp((x_i - x_j) / T),
  translation invariance, and the sum 1;
* the theorem of speculative sampling: one chain step outputs a token
  distributed exactly as p (to the 2^-24 resolution of the random words),
  whatever q is, and its acceptance rate is sum min(p, q) = 1 - TV, the
  pages' identity; both counted exhaustively over all 2^24 values of each
  random word with the oracle's own decision functions;
* closed cases: p == q always accepts, disjoint one-hot rows always reject
  and resample the target token, a draft outside the vocabulary is
  rejected, zero probability is never drawn or accepted;
* the greedy path (temperature 0) equal to the greedy accept oracle;
* compaction invariance: compact accept with length l agrees with the
  full-width (static) accept under the same random words wherever the
  static chain stops before l - 1 ([CSSD], compact vs static);
* the validator: the oracle's own outputs pass it with no band case, and
  outputs with a planted wrong decision or draw fail it;
* the error bounds the validator's band is built from: EPS_W against the
  kernels' stated weight arithmetic taken exactly in rationals, and
  prob_error_bound against weights pushed to the edges of their error.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import sampling as S


def test_softmax_closed_forms():
    x = np.zeros(37, np.float32)
    assert np.allclose(S.softmax64(x, 0.7), 1.0 / 37, rtol=0, atol=1e-17)
    T = np.float32(1.3)
    x2 = np.array([0.0, -np.float64(T) * math.log(3.0)], np.float32)
    p = S.softmax64(x2, T)
    assert abs(p[0] - 0.75) < 1e-7 and abs(p[1] - 0.25) < 1e-7  # x2 rounded to float32
    rng = np.random.default_rng(1)
    # 1/256 steps: adding 8 below is exact in float32
    x = (np.round(rng.normal(0, 3, 2000) * 256) / 256).astype(np.float32)
    for T in (0.3, 1.0, 2.5):
        p = S.softmax64(x, T)
        assert abs(p.sum() - 1.0) < 1e-13
        i, j = np.argmax(x), 17
        assert abs(p[j] / p[i] - math.exp((float(x[j]) - float(x[i])) / float(np.float32(T)))) \
            < 1e-13
        assert np.allclose(S.softmax64(x + np.float32(8.0), T), p, rtol=1e-12, atol=0)
    y = np.array([1.0, -np.inf, 0.0], np.float32)
    assert S.softmax64(y, 1.0)[1] == 0.0


def test_uniform_word():
    assert S.uniform(0) == 0.0 and S.uniform(255) == 0.0
    assert S.uniform(256) == 2.0**-24 and S.uniform(0xFFFFFFFF) == 1.0 - 2.0**-24


def _count_accept(p_d, q_d):
    """#u in [0, 2^24) accepted: the test is monotone in u, so bisect."""
    if not S.accepts(p_d, q_d, 0.0):
        return 0
    if S.accepts(p_d, q_d, 1.0 - 2.0**-24):
        return 1 << 24
    lo, hi = 0, 1 << 24  # accepts(lo) true, accepts(hi) false
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if S.accepts(p_d, q_d, mid / 2.0**24):
            lo = mid
        else:
            hi = mid
    return hi


def _draw_counts(w):
    """#u in [0, 2^24) drawing each index: draw is monotone in u, so bisect
    for the first u of each index."""
    n = len(w)
    first = []
    for i in range(n + 1):
        lo, hi = 0, 1 << 24
        while lo < hi:  # first u with draw(u) >= i
            mid = (lo + hi) // 2
            if S.draw(w, mid / 2.0**24) >= i:
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
    p, q = S.softmax64(p_row, T), S.softmax64(q_row, T)
    R = S.residual(p, q)
    rho = _draw_counts(R if R.sum() > 0 else p)
    out = np.zeros(V)
    acc_rate = 0.0
    for d in range(V):
        a = _count_accept(p[d], q[d]) / 2**24
        acc_rate += q[d] * a
        out[d] += q[d] * a
        out += q[d] * (1 - a) * rho / 2**24
    assert np.max(np.abs(out - p)) < 2 * 2.0**-24, (out, p)
    assert abs(acc_rate - np.minimum(p, q).sum()) < 2 * 2.0**-24
    assert abs(acc_rate - (1 - 0.5 * np.abs(p - q).sum())) < 2 * 2.0**-24


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
    ra[:] = 0xFFFFFFFF  # the largest U still passes when p == q
    res = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, np.ones(B), ra, rs)
    assert res["num_correct"].tolist() == (lens - 1).tolist()
    # disjoint one-hots: q proposes token 3, p puts all mass on token 7
    tgt[:] = -np.inf
    tgt[:, 7] = 0.0
    drf[:] = -np.inf
    drf[:, 3] = 0.0
    drafts[:] = 3
    ra[:] = 0
    res = S.accept_sampling(B, gamma, tgt, drf, "f32", cu, drafts, np.ones(B), ra, rs)
    assert res["num_correct"].tolist() == [0] * B and res["bonus"].tolist() == [7] * B
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
        p = S.softmax64(tgt_c[cu_c[r] + lens[r] - 1], temps[r])
        assert comp["bonus"][r] == S.draw(p, S.uniform(rs[r, lens[r] - 1]))
    assert stops.any() and (~stops).any()


def test_bad_data_falls_back():
    rng = np.random.default_rng(11)
    B, gamma, V = 5, 3, 20
    lens = np.array([4, 2, 3, 1, 4])
    cu, tgt, drf, drafts, ra, rs = _batch(rng, B, gamma, V, lens)
    temps = np.array([1.0, -1.0, 1.0, np.nan, 0.0], np.float32)
    tiny = np.float32(1e-34)  # below the domain (94548.46 / T overflows float32)
    assert not S.temp_ok(tiny) and S.temp_ok(np.float32(3e-34)) and not S.temp_ok(np.inf)
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
    # counts over all 2^24 values of U are the weight shares, rounded up
    w = np.array([0.0, 3.0, 0.0, 5.0, 0.0])
    counts = _draw_counts(w)
    assert counts[0] == 0 and counts[2] == 0 and counts[4] == 0
    assert counts.sum() == 2**24 and abs(counts[1] - 3 * 2**24 / 8) <= 1
    assert S.draw(w, 0.0) == 1 and S.draw(w, 1.0 - 2.0**-24) == 3
    # min(1, p/q) is 0 when p(d) = 0, whatever q(d) is
    assert _count_accept(0.0, 0.4) == 0 and _count_accept(0.0, 0.0) == 0
    # and 1 when p(d) >= q(d) > 0; half the words when p = q / 2
    assert _count_accept(0.4, 0.4) == 2**24 and _count_accept(0.5, 0.25) == 2**24
    assert _count_accept(0.125, 0.25) == 2**23
    # q(d) = 0 < p(d): always accepted
    assert _count_accept(0.1, 0.0) == 2**24


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


def test_accept_probability_at_a_known_ratio():
    # p(d) / q(d) = 0.6 exactly in the softmaxes: rows [0, ln a] at T = 1
    # for target and draft; words just below and above 0.6 * 2^24 decide
    a_p, a_q = 3.0, 1.0  # p = [1/4, 3/4], q = [1/2, 1/2]: p(1)/q(1) = 1.5, p(0)/q(0) = 0.5
    tgt = np.array([[0.0, math.log(a_p)]], np.float32)
    drf = np.array([[0.0, math.log(a_q)]], np.float32)
    p, q = S.softmax64(tgt[0], 1.0), S.softmax64(drf[0], 1.0)
    ratio = p[0] / q[0]
    assert abs(ratio - 0.5) < 1e-7
    u_hi = int(ratio * 2**24)  # U = u_hi / 2^24 just below the ratio
    assert S.accepts(p[0], q[0], u_hi / 2**24) and not S.accepts(p[0], q[0], (u_hi + 2) / 2**24)
    assert S.accepts(p[1], q[1], 1.0 - 2.0**-24)


def _rand_inputs(seed, B=20, gamma=5, V=400):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, gamma + 2, B)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tgt = rng.normal(0, 2.0, (int(cu[-1]), V)).astype(np.float32)
    drf = np.empty((B * gamma, V), np.float32)
    for r in range(B):
        for k in range(gamma):
            src = tgt[cu[r] + k] if k < lens[r] else rng.normal(0, 2.0, V)
            drf[r * gamma + k] = src + rng.normal(0, 0.6, V)
    drafts = np.argmax(drf, axis=1).reshape(B, gamma).astype(np.int32)
    temps = rng.uniform(0.5, 1.5, B).astype(np.float32)
    temps[0] = 0.0
    ra = rng.integers(0, 2**32, (B, gamma), dtype=np.uint64).astype(np.uint32)
    rs = rng.integers(0, 2**32, (B, gamma + 1), dtype=np.uint64).astype(np.uint32)
    return dict(B=B, gamma=gamma, target_rows=tgt, draft_rows=drf, dtype="f32",
                cu_seqlens=cu, drafts=drafts, temps=temps, rand_accept=ra, rand_sample=rs,
                prefix_lens=rng.integers(1, 100, B))


def test_validator_accepts_the_definition_and_rejects_planted_mistakes():
    args = _rand_inputs(41)
    ref = S.accept_sampling(**args)
    rep = S.validate(**args, got=ref)
    assert rep["failures"] == []
    st = rep["stats"]
    assert st["sampling_requests"] == args["B"] - 1 and st["accept_tests"] > 20
    assert st["accept_band_flips"] == 0
    assert st["draws_p_flips"] == 0 and st["draws_residual_flips"] == 0
    B, gamma = args["B"], args["gamma"]
    cu = args["cu_seqlens"]

    def planted(mut):
        g = {k: np.array(v, copy=True) for k, v in ref.items() if k != "status"}
        mut(g)
        return S.validate(**args, got=g)["failures"]

    # one more (or one fewer) accepted draft than the definition gives, where
    # the decision is far from its threshold
    r_rej = next(r for r in range(1, B) if ref["num_correct"][r] < cu[r + 1] - cu[r] - 1)
    def accept_more(g, r=r_rej):
        c = int(g["num_correct"][r]) + 1
        g["num_correct"][r], g["commit"][r] = c, c + 1
        g["new_seq"][r] += 1
        g["out_tokens"][r, :gamma] = args["drafts"][r]
        g["out_tokens"][r, gamma] = -1
        g["out_tokens"][r, c] = g["bonus"][r]
    assert planted(accept_more)
    # a bonus token other than the inverse-CDF one
    def other_bonus(g, r=r_rej):
        b = (int(g["bonus"][r]) + 1) % args["target_rows"].shape[1]
        g["bonus"][r] = b
        g["out_tokens"][r, g["num_correct"][r]] = b
    assert planted(other_bonus)
    # a wrong commit length or new sequence length
    assert planted(lambda g: g["commit"].__setitem__(3, g["commit"][3] + 1))
    assert planted(lambda g: g["new_seq"].__setitem__(4, g["new_seq"][4] - 1))
    # the greedy request (temperature 0) must match exactly
    assert planted(lambda g: g["bonus"].__setitem__(0, g["bonus"][0] + 1))


def test_validator_band_accepts_a_flip_only_near_the_threshold():
    # one request, one draft, p(d) / q(d) = 1/2: a word at U just below 1/2
    # accepts; the validator tolerates the reject decision only while U lies
    # within the band of the threshold
    V = 2
    tgt = np.array([[0.0, math.log(3.0)], [0.0, 0.0]], np.float32)
    drf = np.array([[0.0, 0.0]], np.float32)
    p, q = S.softmax64(tgt[0], 1.0), S.softmax64(drf[0], 1.0)
    eps_p, eta_p = S.prob_error_bound(V)
    base = dict(B=1, gamma=1, target_rows=tgt, draft_rows=drf, dtype="f32",
                cu_seqlens=np.array([0, 2], np.int32), drafts=np.array([[0]], np.int32),
                temps=np.ones(1, np.float32), rand_sample=np.zeros((1, 2), np.uint32))
    rej = {"num_correct": np.array([0]), "bonus": np.array([1]), "commit": np.array([1]),
           "new_seq": np.array([1]), "out_tokens": np.array([[1, -1]])}
    for U, tolerated in ((p[0] / q[0] - 1e-9, True), (p[0] / q[0] - 1e-3, False)):
        w = np.array([[int(U * 2**24) << 8]], np.uint32)
        assert S.accepts(p[0], q[0], S.uniform(w[0, 0]))
        rep = S.validate(**base, rand_accept=w, got=rej)
        assert (rep["failures"] == []) == tolerated, rep
        if tolerated:
            assert rep["stats"]["accept_band"] == 1
    assert eps_p < 1e-4


def test_rejection_draws_from_the_residual_not_from_p():
    # p = [1/2, 1/2], q = [9/10, 1/10]; draft 0 passes with probability 5/9.
    # Rejected, the token comes from max(0, p - q) = [0, 2/5]: always token 1,
    # where a draw from p with the same word (U = 0) would give token 0.
    tgt = np.array([[0.0, 0.0], [0.0, 0.0]], np.float32)
    drf = np.array([[math.log(9.0), 0.0]], np.float32)
    cu = np.array([0, 2], np.int32)
    for w_acc, expect_c in ((np.uint32(0xFFFFFFFF), 0), (np.uint32(0), 1)):
        res = S.accept_sampling(1, 1, tgt, drf, "f32", cu, np.array([[0]], np.int32),
                                np.ones(1, np.float32), np.array([[w_acc]], np.uint32),
                                np.zeros((1, 2), np.uint32))
        assert res["num_correct"][0] == expect_c
        if expect_c == 0:
            assert res["bonus"][0] == 1
        else:  # both passed: the bonus is drawn from p of row 1 with U = 0
            assert res["bonus"][0] == 0


def test_each_draft_is_tested_with_its_own_word():
    # two drafts with p(d) / q(d) = 1/2 each: word 0 (U = 0) passes, the
    # largest word rejects; the first rejected draft names the word used
    tgt = np.array([[0.0, 0.0]] * 3, np.float32)  # p = [1/2, 1/2]
    drf = np.array([[0.0, -np.inf]] * 2, np.float32)  # q = [1, 0]: p(0) / q(0) = 1/2
    cu = np.array([0, 3], np.int32)
    drafts = np.array([[0, 0]], np.int32)
    hi = np.uint32(0xFFFFFFFF)
    for ra, expect in (([0, hi], 1), ([hi, 0], 0), ([0, 0], 2)):
        res = S.accept_sampling(1, 2, tgt, drf, "f32", cu, drafts, np.ones(1, np.float32),
                                np.array([ra], np.uint32), np.zeros((1, 3), np.uint32))
        assert res["num_correct"][0] == expect


# ---- the per-weight bound EPS_W against the kernels' stated weight arithmetic


def _round_f32(fr):
    """The float32 nearest to the rational fr (ties to even), as a Fraction;
    normal range only."""
    from fractions import Fraction
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # 24 significant bits: a = m * 2^(e - 23), m in [2^23, 2^24)
    scale = Fraction(2) ** (23 - e)
    m = a * scale
    q, rem = divmod(m.numerator, m.denominator)
    half = Fraction(rem, m.denominator)
    if half > Fraction(1, 2) or (half == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return sign * Fraction(q) / scale


def test_eps_w_covers_the_kernels_weight_arithmetic():
    """W = nearest integer to 2^t, t = RN32((x - m) c' + 31) in one fused
    multiply-add, c' = RN32(K / T) 2^-16, K = RN32(2^16 log2 e), with 2^t off
    by up to one float32 unit either way: |W - W*| <= EPS_W W* + 1/2 + 1e-5
    for W* = 2^31 exp((x - m) / T), over random rows, temperatures and float32
    or bfloat16 values (the fused multiply-add and every rounding taken
    exactly, in rationals)."""
    from fractions import Fraction
    rng = np.random.default_rng(77)
    K = Fraction(float(np.float32(94548.4609375)))
    worst = 0.0
    for _ in range(3000):
        T = np.float32(np.exp(rng.uniform(np.log(0.02), np.log(8.0))))
        m = np.float32(rng.normal(0, 20))
        # t* spread over [-2, 31]
        ts = rng.uniform(-2.0, 31.0)
        x = np.float32(m + (ts - 31.0) * float(T) / math.log2(math.e))
        if rng.random() < 0.5:  # bfloat16 values
            x = np.float32(np.frombuffer((np.float32(x).view(np.uint32) & 0xFFFF0000).tobytes(),
                                         np.float32)[0])
            m = np.float32(np.frombuffer((np.float32(m).view(np.uint32) & 0xFFFF0000).tobytes(),
                                         np.float32)[0])
        if x > m:
            x, m = m, x
        c = _round_f32(K / Fraction(float(T))) / 2**16
        d = _round_f32(Fraction(float(x)) - Fraction(float(m)))
        t = float(_round_f32(d * c + 31))
        y = 2.0 ** t
        ws = 2.0**31 * math.exp((float(x) - float(m)) / float(T))
        ulp = 2.0 ** (math.frexp(y)[1] - 24)
        for yh in (y - ulp, y, y + ulp):
            W = float(np.rint(yh))
            assert abs(W - ws) <= S.EPS_W * ws + 0.5 + 1e-5, (float(x), float(m), float(T), W, ws)
            if ws > 1e6:  # the relative part, net of the half unit
                worst = max(worst, (abs(W - ws) - 0.5) / ws)
    # random rows reach a fair part of the worst case (about a quarter)
    assert worst > 0.1 * S.EPS_W, worst


@pytest.mark.parametrize("V", [7, 1000, 32000, 151936])
def test_prob_error_bound_covers_weights_at_the_edges_of_their_error(V):
    """prob_error_bound against weights W = W* (1 + e) + a pushed to the edges
    of the per-weight model (|e| = EPS_W, |a| = 1/2, W >= 0): the token under
    test pushed up or down and every other weight the other way. Every token's
    probability stays within eps_p p + eta_p of the float64 softmax, on
    workload-like rows and on rows built to make the bound tight (one maximum
    and V - 1 weights of 1 to 3 units, so the half units add up in the
    normaliser); there the worst case reaches over 90% of the bound, so a term
    dropped from it fails."""
    rng = np.random.default_rng(V)
    eps_p, eta_p = S.prob_error_bound(V)
    a = 0.5
    rows = [rng.normal(0.0, 3.0, V), rng.standard_cauchy(V).clip(-60, 60)]
    tight = np.log(rng.uniform(1.0, 3.0, V) / 2.0**31)
    tight[rng.integers(V)] = 0.0
    rows.append(tight)
    worst = 0.0
    for k, x in enumerate(rows):
        ws = 2.0**31 * np.exp(x - x.max())
        p = ws / ws.sum()
        for i in {int(np.argmax(x)), int(rng.integers(V)), int(np.argmin(x))}:
            for sgn in (1.0, -1.0):
                e = np.full(V, -sgn * S.EPS_W)
                off = np.full(V, -sgn * a)
                e[i], off[i] = sgn * S.EPS_W, sgn * a
                W = np.maximum(ws * (1.0 + e) + off, 0.0)
                pp = W / W.sum()
                ratio = np.abs(pp - p) / (eps_p * p + eta_p)
                assert ratio.max() <= 1.0, (k, i, sgn, float(ratio.max()))
                if k == 2:
                    worst = max(worst, float(ratio[i]))
    assert worst > 0.9, worst
