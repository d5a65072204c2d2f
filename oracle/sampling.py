"""Chain speculative-sampling accept oracle, the float64 definition. TEST
INFRASTRUCTURE ONLY.

What the pages fix:

* [Round] §五 (AcceptSampling): the sampling path accepts or rejects each
  draft by speculative sampling over the draft-side probabilities that
  actually proposed it and the target probabilities, not by token equality;
  it yields correct_len and a bonus token, and the bonus source moves with
  the acceptance end point as in the greedy path.
* [Budget] §二: a draft x drawn from q is accepted with probability
  min(1, p(x) / q(x)), so the mean acceptance is sum_x min(p(x), q(x)) =
  1 - TV(q, p).
* [CSSD] "截短为什么不会改变目标分布": the scheduler only chooses the
  candidate set; accept, reject and the residual resample follow the
  speculative algorithm, and the random numbers must keep their meaning
  under batch compaction. "常见失败模式": compact and static must agree
  under the same random conditions.

The rest is the standard chain rule of speculative sampling, written here
in float64 in the pages' terms. For request r with verify length l (rows
0..l-1 of its packed block) at temperature T > 0:

* p_j = softmax(x / T) of target row j, q_k = softmax(x / T) of the draft
  row that proposed draft k (row r * gamma + k - 1); float32 logits
  (bfloat16 widens exactly), the softmax in float64 with the row maximum
  subtracted.
* Drafts k = 1..l-1 in order: draft d is accepted iff U < p_{k-1}(d) /
  q_k(d), written U * q_k(d) < p_{k-1}(d) (so a draft with q(d) = 0 passes
  iff p(d) > 0, and one with p(d) = 0 never passes). A draft outside [0, V)
  is rejected.
* The first rejected draft k ends the chain with correct = k - 1; the token
  of output column k - 1 is drawn from the residual max(0, p_{k-1} - q_k),
  normalised (from p_{k-1} if the residual is 0 everywhere). If every draft
  passes, the token of column l - 1 is drawn from p_{l-1}.
* Readings where the pages give no rule (also in the design notes): the
  caller passes 32-bit random words keyed by (request, position), a word w
  standing for U = (w >> 8) / 2^24: ``rand_accept[r, k-1]`` tests draft k,
  ``rand_sample[r, c]`` draws the token of column c. A draw from weights w
  takes the smallest index i with cumsum(w)_i > U * sum(w) (inverse CDF).
* Temperature 0 marks a greedy request: the greedy rule of
  ``oracle.accept`` applies. A temperature that is negative, NaN or
  infinite, or below the domain the kernels accept (the float32 quotient
  94548.4609375 / T overflows, T below about 2.8e-34),
  sets DATA_BAD_CONF; a NaN or +inf logit, or no finite element, in a row
  a sampling request reads sets DATA_BAD_LOGITS. Either way the request
  gets the malformed-layout outputs of ``oracle.accept`` (correct 0, bonus
  -1, commit 0, out_tokens -1, new_seq = prefix).

An implementation that takes p and q at a finite resolution decides
differently from this definition only where U lies within that
resolution's error of a threshold. ``validate`` checks such an
implementation's outputs: every decision must equal this definition's
unless U lies inside the band the stated per-token error allows, and the
chain then continues along the implementation's decision. The band follows
from a per-token bound |p'(i) - p(i)| <= eps_p * p(i) + eta_p (see
``prob_error_bound``).
"""

from __future__ import annotations

import math

import numpy as np

from .accept import as_f32_rows, row_argmax
from .pack import DATA_BAD_LENS
from .plan import DATA_BAD_CONF

DATA_BAD_LOGITS = 8
WORD_SHIFT = 8  # a word w stands for U = (w >> 8) / 2^24
U_SCALE = float(1 << 24)
# The largest relative error of one unnormalised weight of the kernels, before
# its rounding to an integer. The kernels form t = RN32((x - m) c' + 31) with
# c' = RN32(K / T) 2^-16 and K = RN32(2^16 log2 e) in one fused multiply-add,
# and 2^t with the hardware exponential; the exact exponent is
# t* = 31 + (x - m) log2(e) / T. For every weight of at least 1/2
# (|t* - 31| <= 32):
#   |t - t*| <= 32 (2^-24 [x - m] + 2^-24 [K / T] + 1.34e-8 [K]) + 2^-20
#             = 5.20e-6 (in base-2 units), a relative 3.61e-6 on 2^t;
#   the exponential itself: within one float32 unit, 2^-23 = 1.19e-7
#   relative (0.79 units measured on gfx950);
# together 3.73e-6, rounded up. Smaller weights are within their own size
# of 0, inside the absolute term of ``prob_error_bound``.
EPS_W = 4.0e-6


def uniform(word) -> float:
    """U = (word >> 8) / 2^24, in [0, 1 - 2^-24]."""
    return float(int(word) >> WORD_SHIFT) / U_SCALE


def row_is_bad(x: np.ndarray) -> bool:
    """NaN or +inf anywhere, or no finite maximum."""
    x = np.asarray(x, dtype=np.float32)
    if np.isnan(x).any() or np.isposinf(x).any():
        return True
    return not np.isfinite(np.max(x))


def temp_ok(T) -> bool:
    """A sampling temperature inside the domain: positive, finite, and not so
    small that the float32 quotient 94548.4609375 / T overflows."""
    T32 = np.float32(T)
    if not (T32 > 0 and np.isfinite(T32)):
        return False
    with np.errstate(over="ignore"):
        return bool(np.isfinite(np.float32(94548.4609375) / T32))


def softmax64(x, T) -> np.ndarray:
    """softmax(x / T) in float64 of one float32 row, the maximum subtracted."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    y = (x - np.max(x)) / np.float64(np.float32(T))
    e = np.exp(y)
    return e / np.sum(e)


def accepts(p_d: float, q_d: float, U: float) -> bool:
    """U < p(d) / q(d), written without a division."""
    return U * q_d < p_d


def residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """max(0, p - q), unnormalised."""
    return np.maximum(p - q, 0.0)


def draw(w: np.ndarray, U: float) -> int:
    """Inverse CDF: the smallest i with cumsum(w)_i > U * sum(w)."""
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    return int(np.searchsorted(c, U * c[-1], side="right"))


def accept_sampling(B, gamma, target_rows, draft_rows, dtype, cu_seqlens, drafts, temps,
                    rand_accept, rand_sample, prefix_lens=None, max_rows=None):
    """Chain speculative-sampling accept over packed target rows, float64.

    target_rows [>= cu[B], V] and draft_rows [B * gamma, V] (row r * gamma +
    k - 1 proposed draft k) as float32, or bfloat16 bit patterns with
    dtype "bf16". Returns num_correct, bonus, commit, new_seq, out_tokens
    and status."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    drafts = np.asarray(drafts, dtype=np.int64).reshape(B, gamma)
    temps = np.asarray(temps, dtype=np.float32).reshape(B)
    ra = np.asarray(rand_accept, dtype=np.uint32).reshape(B, gamma)
    rs = np.asarray(rand_sample, dtype=np.uint32).reshape(B, gamma + 1)
    prefix = np.zeros(B, np.int64) if prefix_lens is None else np.asarray(prefix_lens, np.int64)
    tgt = as_f32_rows(target_rows, dtype)
    dr = as_f32_rows(draft_rows, dtype)
    V = tgt.shape[1]
    total = int(cu[B]) if B > 0 else 0
    limit = min(total, tgt.shape[0] if max_rows is None else max_rows)
    correct = np.zeros(B, np.int32)
    bonus = np.full(B, -1, np.int32)
    commit = np.zeros(B, np.int32)
    out = np.full((B, gamma + 1), -1, np.int32)
    status = 0
    for r in range(B):
        s, e = int(cu[r]), int(cu[r + 1])
        l = e - s
        if not (1 <= l <= gamma + 1 and 0 <= s and e <= limit):
            status |= DATA_BAD_LENS
            continue
        T = float(temps[r])
        if T == 0.0:
            am = row_argmax(tgt[s:e])
            c = 0
            while c < l - 1 and drafts[r, c] == am[c]:
                c += 1
            tok = int(am[c])
        elif not temp_ok(T):
            status |= DATA_BAD_CONF
            continue
        else:
            rows = [tgt[s + j] for j in range(l)] + [dr[r * gamma + k] for k in range(l - 1)]
            if any(row_is_bad(x) for x in rows):
                status |= DATA_BAD_LOGITS
                continue
            c, tok = l - 1, None
            for k in range(1, l):
                p = softmax64(tgt[s + k - 1], T)
                q = softmax64(dr[r * gamma + k - 1], T)
                d = int(drafts[r, k - 1])
                if 0 <= d < V and accepts(p[d], q[d], uniform(ra[r, k - 1])):
                    continue
                R = residual(p, q)
                c, tok = k - 1, draw(R if R.sum() > 0 else p, uniform(rs[r, k - 1]))
                break
            if tok is None:
                tok = draw(softmax64(tgt[s + l - 1], T), uniform(rs[r, l - 1]))
        correct[r] = c
        bonus[r] = tok
        commit[r] = c + 1
        out[r, :gamma] = drafts[r]
        out[r, gamma] = -1
        out[r, c] = tok
    return {"num_correct": correct, "bonus": bonus, "commit": commit,
            "new_seq": (prefix + commit).astype(np.int32), "out_tokens": out, "status": status}


# ---------------------------------------------------------------- validation


def prob_error_bound(V: int, eps_w: float = EPS_W):
    """(eps_p, eta_p) with |p'(i) - p(i)| <= eps_p * p(i) + eta_p for every
    token of a V-token row, when p' = W / sum W is formed from weights
    W_i = W*_i (1 + e_i) + a_i, |e_i| <= eps_w and |a_i| <= 1/2 + 1e-5 (a
    rounding to the nearest integer, the weights below 1/2 included), around exact
    weights W*_i = 2^31 exp((x_i - m) / T) whose sum is at least 2^31 (the
    maximum's own weight).

    With the normaliser's relative error zeta = eps_w + a * V / 2^31:
    p'/p - 1 = (1 + e_i) / (1 + zeta_Z) - 1 - ..., so
    eps_p = (eps_w + zeta) / (1 - zeta) and eta_p = a / (2^31 (1 - zeta))."""
    a = 0.5 + 1e-5
    zeta = eps_w + a * V / 2.0**31
    return (eps_w + zeta) / (1.0 - zeta), a / (2.0**31 * (1.0 - zeta))


def _draw_check(w, U, g, delta, n):
    """Is token g a valid draw for U when every CDF value may be off by delta?
    Returns (float64 token k, U within delta of a boundary of k's CDF step,
    ok)."""
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    S = c[-1]
    k = int(np.searchsorted(c, U * S, side="right"))
    near = U - (c[k - 1] / S if k > 0 else 0.0) <= delta or c[k] / S - U <= delta
    if g == k:
        return k, near, True
    if not (0 <= g < n):
        return k, near, False
    lo = (c[g - 1] / S if g > 0 else 0.0) - delta
    hi = c[g] / S + delta
    slack = 1e-12
    ok = lo - slack <= U <= hi + slack
    return k, near, ok


def validate(B, gamma, target_rows, draft_rows, dtype, cu_seqlens, drafts, temps, rand_accept,
             rand_sample, got, prefix_lens=None, max_rows=None, reqs=None, eps_w=EPS_W):
    """Check an implementation's outputs ``got`` (num_correct, bonus, commit,
    new_seq, out_tokens as arrays over all B requests) against the float64
    definition, request by request (all, or those listed in ``reqs``).

    Greedy, malformed and out-of-domain requests must match exactly. For a
    sampling request the chain is walked in float64 along the
    implementation's own decisions:

    * accept test of draft d with U: the margin g = U q(d) - p(d) decides
      (accept iff g < 0). With p', q' within the bound of
      ``prob_error_bound``, the implementation's margin differs from g by at
      most band = eps_p (p(d) + U q(d)) + 2 eta_p, so its decision must
      equal the float64 one when |g| > band; otherwise the case is counted
      as a band case and either decision is valid;
    * the draw: the implementation's token must be the float64 inverse-CDF
      token unless U lies within delta of a CDF boundary, where delta =
      eps_p + V eta_p for a draw from p; for the residual, whose total R
      (= TV) and partial sums each move by at most E = 2 eps_p + 2 V eta_p,
      delta = 2 E / (R - E) (every token of positive weight is valid when
      R <= E). The token must still fall inside its own widened CDF step.

    Returns a dict of counts (accept tests and draws; of each, how many had
    U inside the band and how many of those the implementation decided
    differently from float64: the flips) and a list of failure strings
    (empty when valid)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    drafts = np.asarray(drafts, dtype=np.int64).reshape(B, gamma)
    temps = np.asarray(temps, dtype=np.float32).reshape(B)
    ra = np.asarray(rand_accept, dtype=np.uint32).reshape(B, gamma)
    rs = np.asarray(rand_sample, dtype=np.uint32).reshape(B, gamma + 1)
    prefix = np.zeros(B, np.int64) if prefix_lens is None else np.asarray(prefix_lens, np.int64)
    tgt = as_f32_rows(target_rows, dtype)
    dr = as_f32_rows(draft_rows, dtype)
    V = tgt.shape[1]
    eps_p, eta_p = prob_error_bound(V, eps_w)
    total = int(cu[B]) if B > 0 else 0
    limit = min(total, tgt.shape[0] if max_rows is None else max_rows)
    g_nc = np.asarray(got["num_correct"])
    g_bo = np.asarray(got["bonus"])
    g_cm = np.asarray(got["commit"])
    g_ns = np.asarray(got["new_seq"])
    g_out = np.asarray(got["out_tokens"]).reshape(-1, gamma + 1)
    stats = {"requests": 0, "sampling_requests": 0, "accept_tests": 0, "accept_band": 0,
             "accept_band_flips": 0, "draws_p": 0, "draws_p_band": 0, "draws_p_flips": 0,
             "draws_residual": 0, "draws_residual_band": 0, "draws_residual_flips": 0,
             "accept_min_rel_margin": math.inf}
    fails = []

    def expect(r, c, tok):
        want_out = np.array(drafts[r].tolist() + [-1], np.int64)
        if tok is not None:
            want_out[c] = tok
        if not (g_nc[r] == c and g_bo[r] == tok and g_cm[r] == c + 1
                and g_ns[r] == prefix[r] + c + 1 and np.array_equal(g_out[r], want_out)):
            fails.append(f"r={r}: outputs ({g_nc[r]}, {g_bo[r]}, {g_cm[r]}, {g_ns[r]}) "
                         f"!= expected ({c}, {tok}, {c + 1}, {prefix[r] + c + 1}) or out_tokens")

    def expect_bad(r):
        if not (g_nc[r] == 0 and g_bo[r] == -1 and g_cm[r] == 0 and g_ns[r] == prefix[r]
                and np.all(g_out[r] == -1)):
            fails.append(f"r={r}: expected the malformed-request outputs")

    for r in (range(B) if reqs is None else reqs):
        r = int(r)
        stats["requests"] += 1
        s, e = int(cu[r]), int(cu[r + 1])
        l = e - s
        if not (1 <= l <= gamma + 1 and 0 <= s and e <= limit):
            expect_bad(r)
            continue
        T = float(temps[r])
        if T == 0.0:
            am = row_argmax(tgt[s:e])
            c = 0
            while c < l - 1 and drafts[r, c] == am[c]:
                c += 1
            expect(r, c, int(am[c]))
            continue
        rows = [tgt[s + j] for j in range(l)] + [dr[r * gamma + k] for k in range(l - 1)]
        if not temp_ok(T) or any(row_is_bad(x) for x in rows):
            expect_bad(r)
            continue
        stats["sampling_requests"] += 1
        gc = int(g_nc[r])
        if not 0 <= gc <= l - 1:
            fails.append(f"r={r}: num_correct {gc} outside [0, {l - 1}]")
            continue
        chain_ok = True
        for k in range(1, gc + 2 if gc < l - 1 else l):
            p = softmax64(tgt[s + k - 1], T)
            q = softmax64(dr[r * gamma + k - 1], T)
            d = int(drafts[r, k - 1])
            U = uniform(ra[r, k - 1])
            gpu_acc = k <= gc
            stats["accept_tests"] += 1
            if not 0 <= d < V:
                if gpu_acc:
                    fails.append(f"r={r} k={k}: draft {d} outside the vocabulary accepted")
                    chain_ok = False
                    break
                f64_acc = False
                band = False
            else:
                marg = U * q[d] - p[d]
                width = eps_p * (p[d] + U * q[d]) + 2.0 * eta_p
                f64_acc = marg < 0.0
                band = abs(marg) <= width
                if p[d] + U * q[d] > 0:
                    stats["accept_min_rel_margin"] = min(stats["accept_min_rel_margin"],
                                                         abs(marg) / (p[d] + U * q[d]))
            if band:
                stats["accept_band"] += 1
                stats["accept_band_flips"] += int(gpu_acc != f64_acc)
            elif gpu_acc != f64_acc:
                fails.append(f"r={r} k={k}: accept {gpu_acc} but float64 says {f64_acc} "
                             f"(U={U:.9f}, p={p[d] if 0 <= d < V else 0:.6g}, "
                             f"q={q[d] if 0 <= d < V else 0:.6g})")
                chain_ok = False
                break
            if not gpu_acc:  # the chain ends with a residual draw
                R = residual(p, q)
                Rs = float(R.sum())
                E = 2.0 * eps_p + 2.0 * V * eta_p
                Us = uniform(rs[r, k - 1])
                stats["draws_residual"] += 1
                if Rs == 0.0:
                    ex_tok, near, ok = _draw_check(p, Us, int(g_bo[r]), eps_p + V * eta_p, V)
                elif Rs <= E:  # any token the residual or p could hold
                    ex_tok, near, ok = draw(R, Us), True, 0 <= int(g_bo[r]) < V
                else:
                    ex_tok, near, ok = _draw_check(R, Us, int(g_bo[r]), 2.0 * E / (Rs - E), V)
                stats["draws_residual_band"] += int(near)
                stats["draws_residual_flips"] += int(ok and ex_tok != int(g_bo[r]))
                if not ok:
                    fails.append(f"r={r} k={k}: residual draw {int(g_bo[r])}, float64 gives "
                                 f"{ex_tok} (U={Us:.9f}, TV={Rs:.6g})")
                    chain_ok = False
                break
        if not chain_ok:
            continue
        if gc == l - 1:  # every draft passed: the bonus is drawn from p of row l-1
            p = softmax64(tgt[s + l - 1], T)
            Us = uniform(rs[r, l - 1])
            ex_tok, near, ok = _draw_check(p, Us, int(g_bo[r]), eps_p + V * eta_p, V)
            stats["draws_p"] += 1
            stats["draws_p_band"] += int(near)
            stats["draws_p_flips"] += int(ok and ex_tok != int(g_bo[r]))
            if not ok:
                fails.append(f"r={r}: bonus draw {int(g_bo[r])}, float64 gives {ex_tok} "
                             f"(U={Us:.9f})")
                continue
        expect(r, gc, int(g_bo[r]))
    return {"stats": stats, "failures": fails}
