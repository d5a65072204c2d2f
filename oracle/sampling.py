"""Chain speculative-sampling accept oracle. TEST INFRASTRUCTURE ONLY.

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

The rest is the standard chain rule of speculative sampling, stated here in
the pages' terms. For request r with verify length l (rows 0..l-1 of its
packed block), drafts k = 1..l-1 are tested in order: draft k against target
row k-1 (p) and draft row k-1 (q, the distribution that proposed it). The
first rejected draft k ends the chain with correct = k - 1, and the token at
output column k - 1 is drawn from the residual max(0, p - q) of that pair. If
all l - 1 drafts pass, the token at column l - 1 is drawn from p of target
row l - 1. A temperature of 0 marks a greedy request: the greedy rule of
``oracle.accept`` applies to it.

Readings (also in the design notes), chosen so that every decision is an
exact integer comparison, identical on any device and in any summation
order:

* Probabilities at fixed resolution. For a row x (float32; bfloat16 widens
  exactly) at temperature T > 0, with m = max x:
      t_i = RN64(RN64(m - x_i) * RN64(65536 / T)),   j_i = nearest integer
      (ties to even), and W_i = 0 when t_i or j_i >= 455 * 4096; otherwise
      P = (E0[j >> 12] * E1[(j >> 6) & 63] + 2^22) >> 23
      W = (P * E2[j & 63] + 2^22) >> 23
  with E0[h] = round(2^40 e^(-h/16)) (h < 455), E1[a] = round(2^23
  e^(-a/1024)) and E2[b] = round(2^23 e^(-b/65536)) (a, b < 64), each the
  nearest integer to the real value. So W_i ~ 2^40 exp((x_i - m) / T) within
  about 8e-6 relative, W = 2^40 at the maximum, and p_i = W_i / Z with
  Z = sum W (an integer below 2^58).
* Random words. The caller passes 32-bit words; a word w stands for the
  uniform U = (w >> 8) / 2^24. ``rand_accept[r, k-1]`` tests draft k;
  ``rand_sample[r, c]`` draws the token of output column c. Keying them by
  (request, position) keeps their meaning under compaction.
* Accept draft d iff u * Wq[d] * Zp < 2^24 * Wp[d] * Zq (u = w >> 8), which
  is U < p(d) / q(d), i.e. the min(1, p/q) rule. A draft outside [0, V) has
  Wp = Wq = 0 and is rejected.
* Drawing from integer weights w (total S) with word v: the smallest i whose
  running sum exceeds floor((v >> 8) * S / 2^24).
* The residual weights are R_i = max(0, Wp_i * Zq - Wq_i * Zp) (that is
  max(0, p - q) scaled by Zp * Zq). If they are all 0 (p == q at this
  resolution and the draft had zero weight on both sides), the token is
  drawn from p.
* A row with a NaN or +inf logit, or with no finite maximum, in a sampling
  request sets DATA_BAD_LOGITS; a temperature that is negative, NaN or
  infinite sets DATA_BAD_CONF. Either way the request gets the malformed-
  layout outputs of ``oracle.accept`` (correct 0, bonus -1, commit 0,
  out_tokens -1, new_seq = prefix). Greedy requests follow ``oracle.accept``
  in full, NaN ordering included.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from .accept import as_f32_rows, row_argmax
from .pack import DATA_BAD_LENS
from .plan import DATA_BAD_CONF

DATA_BAD_LOGITS = 8
E0_LEN = 455
J_MAX = E0_LEN * 4096

_TABLES = None


def _nearest_int_exp(num: int, den: int, scale_log2: int) -> int:
    """Nearest integer to 2**scale_log2 * exp(-num/den), from the exact
    rational Taylor series of exp(num/den) with a bound on its remainder."""
    x = Fraction(num, den)
    if num == 0:
        return 1 << scale_log2
    term, total, n = Fraction(1), Fraction(1), 0
    while True:
        n += 1
        term = term * x / n
        total += term
        # once the terms decrease, the remainder is below term * x / (n + 1 - x)
        if n + 1 > 2 * x:
            rem = term * x / (n + 1 - x)
            lo = Fraction(1 << scale_log2) / (total + rem)
            hi = Fraction(1 << scale_log2) / total
            a, b = lo - Fraction(1, 2), hi - Fraction(1, 2)
            # nearest integer of every value in [lo, hi] is the same
            if a.__ceil__() == b.__ceil__() and a != a.__ceil__() and b != b.__ceil__():
                return int(a.__ceil__())


def exp_tables():
    """(E0, E1, E2) as lists of Python ints, computed once."""
    global _TABLES
    if _TABLES is None:
        e0 = [_nearest_int_exp(h, 16, 40) for h in range(E0_LEN)]
        e1 = [_nearest_int_exp(a, 1024, 23) for a in range(64)]
        e2 = [_nearest_int_exp(b, 65536, 23) for b in range(64)]
        _TABLES = (e0, e1, e2)
    return _TABLES


def row_is_bad(x: np.ndarray) -> bool:
    """NaN or +inf anywhere, or no finite maximum."""
    x = np.asarray(x, dtype=np.float32)
    if np.isnan(x).any() or np.isposinf(x).any():
        return True
    return not np.isfinite(np.max(x))


def weights(x: np.ndarray, T: float) -> np.ndarray:
    """Integer weights W (uint64) of one float32 row at temperature T > 0."""
    e0, e1, e2 = (np.array(t, dtype=np.uint64) for t in exp_tables())
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    m = np.max(x)
    s = np.float64(65536.0) / np.float64(np.float32(T))
    with np.errstate(invalid="ignore", over="ignore"):
        t = (m - x) * s  # two float64 roundings, as in the definition
    W = np.zeros(x.shape, dtype=np.uint64)
    ok = t < J_MAX
    j = np.rint(t[ok]).astype(np.int64)
    keep = j < J_MAX
    j = j[keep]
    P = (e0[j >> 12] * e1[(j >> 6) & 63] + np.uint64(1 << 22)) >> np.uint64(23)
    w = (P * e2[j & 63] + np.uint64(1 << 22)) >> np.uint64(23)
    idx = np.flatnonzero(ok)[keep]
    W[idx] = w
    return W


def draw(w, word: int) -> int:
    """Smallest i whose running sum of the integer weights w exceeds
    floor((word >> 8) * sum(w) / 2**24)."""
    w = np.asarray(w, dtype=object)
    S = int(np.sum(w))
    t = ((int(word) >> 8) * S) >> 24
    cum = np.cumsum(w)
    return int(np.argmax(cum > t))


def accepts(Wp_d: int, Zp: int, Wq_d: int, Zq: int, word: int) -> bool:
    """U < p(d) / q(d) with U = (word >> 8) / 2**24, in integers."""
    return (int(word) >> 8) * int(Wq_d) * int(Zp) < (1 << 24) * int(Wp_d) * int(Zq)


def residual(Wp: np.ndarray, Zp: int, Wq: np.ndarray, Zq: int) -> np.ndarray:
    """max(0, Wp * Zq - Wq * Zp) as Python ints."""
    d = Wp.astype(object) * int(Zq) - Wq.astype(object) * int(Zp)
    return np.where(d > 0, d, 0)


def sample_pair(p_row, q_row, T, d, u_word, v_word, V=None):
    """One chain step on float32 rows: (accepted, token drawn if rejected)."""
    Wp, Wq = weights(p_row, T), weights(q_row, T)
    Zp, Zq = int(Wp.sum()), int(Wq.sum())
    V = Wp.size if V is None else V
    in_range = 0 <= d < V
    if in_range and accepts(int(Wp[d]), Zp, int(Wq[d]), Zq, u_word):
        return True, None
    R = residual(Wp, Zp, Wq, Zq)
    if int(np.sum(R)) == 0:
        return False, draw(Wp, v_word)
    return False, draw(R, v_word)


def accept_sampling(B, gamma, target_rows, draft_rows, dtype, cu_seqlens, drafts, temps,
                    rand_accept, rand_sample, prefix_lens=None, max_rows=None):
    """Chain speculative-sampling accept over packed target rows.

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
        elif not (T > 0.0 and np.isfinite(T)):
            status |= DATA_BAD_CONF
            continue
        else:
            rows = [tgt[s + j] for j in range(l)] + [dr[r * gamma + k] for k in range(l - 1)]
            if any(row_is_bad(x) for x in rows):
                status |= DATA_BAD_LOGITS
                continue
            c, tok = l - 1, None
            for k in range(1, l):
                ok, t_rej = sample_pair(tgt[s + k - 1], dr[r * gamma + k - 1], T,
                                        int(drafts[r, k - 1]), int(ra[r, k - 1]),
                                        int(rs[r, k - 1]), V)
                if not ok:
                    c, tok = k - 1, t_rej
                    break
            if tok is None:
                tok = draw(weights(tgt[s + l - 1], T), int(rs[r, l - 1]))
        correct[r] = c
        bonus[r] = tok
        commit[r] = c + 1
        out[r, :gamma] = drafts[r]
        out[r, gamma] = -1
        out[r, c] = tok
    return {"num_correct": correct, "bonus": bonus, "commit": commit,
            "new_seq": (prefix + commit).astype(np.int32), "out_tokens": out, "status": status}
