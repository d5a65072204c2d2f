"""Fixed-resolution form of the chain speculative-sampling accept: a
WHITE-BOX check of the kernels, not the definition. TEST INFRASTRUCTURE ONLY.

The definition the pages give is the float64 one in ``oracle.sampling``
(softmax p and q, accept iff U < p(d) / q(d), the residual max(0, p - q)).
This module restates the implementation choice the kernels make on top of
it: p and q taken at a fixed integer resolution, so that every accept test
and every draw is an exact integer decision, reproducible on any device and
in any summation order. GPU results are checked two ways: against the
float64 definition, where every decision must agree except where the random
number lies inside the error band of this resolution (``oracle.sampling.
validate``), and against this module bit for bit, which pins the kernels'
own arithmetic (a weight off by one step changes no decision, but it changes
the sums this module predicts exactly).

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

The fixed-resolution scheme, chosen so that every decision is an exact
integer comparison, identical on any device and in any summation order:

* Probabilities at fixed resolution. For a row x (float32; bfloat16 widens
  exactly) at temperature T > 0, with m = max x, every step one IEEE float32
  operation (nearest, ties to even):
      c = K / T with K = 94548.4609375, the float32 nearest to 2^16 log2(e)
      u_i = (m - x_i) * c            (u ~ 2^16 * (m - x_i) * log2(e) / T)
  then, in integers, W_i = 0 unless j = (nearest integer to u_i, ties to
  even) is below 2^21; else with n = j >> 16, h = (j >> 8) & 255, r = j & 255,
      Y = B[h] - (((B[h] - B[h+1]) * r + 128) >> 8)
      W_i = (Y + (2^n >> 1)) >> n
  where B[i] is the nearest integer to 2^31 * 2^(-i/256) (i = 0..256). So
  W_i ~ 2^31 * 2^(-j/65536) ~ 2^31 exp((x_i - m) / T): the octave n is a
  rounding shift and the fraction a linear interpolation, within about 6e-6
  relative (the 2^-16 step of j and the interpolation) plus half a unit.
  W = 2^31 at the maximum, and p_i = W_i / Z with Z = sum W (below 2^49).
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
  infinite, or so small that K / T overflows float32 (T below about
  2.8e-34), sets DATA_BAD_CONF. Either way the request gets the malformed-
  layout outputs of ``oracle.accept`` (correct 0, bonus -1, commit 0,
  out_tokens -1, new_seq = prefix). Greedy requests follow ``oracle.accept``
  in full, NaN ordering included.
"""

from __future__ import annotations

import numpy as np

from .accept import as_f32_rows, row_argmax
from .pack import DATA_BAD_LENS
from .plan import DATA_BAD_CONF

DATA_BAD_LOGITS = 8
K_LOG2E_16 = np.float32(94548.4609375)  # float32 nearest to 2^16 * log2(e)
J_MAX = 1 << 21
B_LEN = 257

_TABLE = None


def _nearest_int_pow2(e_num: int, e_den: int) -> int:
    """Nearest integer (ties to even) to 2**(e_num / e_den), exactly.

    An integer exponent gives a power of two: 2**-1 = 1/2 is the only tie
    (it goes to 0). Otherwise the value is irrational, so N is the nearest
    integer iff (2N - 1)**e_den < 2**(e_den + e_num) < (2N + 1)**e_den, all
    integers; below 1/2 (e_den + e_num < 0) it is 0."""
    if e_num % e_den == 0:
        k = e_num // e_den
        return 1 << k if k >= 0 else 0
    if e_den + e_num < 0:
        return 0
    target = 1 << (e_den + e_num)
    n = max(0, int(round(2.0 ** (e_num / e_den))))
    while (2 * n + 1) ** e_den <= target:
        n += 1
    while n > 0 and (2 * n - 1) ** e_den >= target:
        n -= 1
    return n


def exp_table():
    """B[i] = nearest integer to 2^31 * 2^(-i/256), i = 0..256 (Python ints)."""
    global _TABLE
    if _TABLE is None:
        _TABLE = [_nearest_int_pow2(31 * 256 - i, 256) for i in range(B_LEN)]
    return _TABLE


def row_is_bad(x: np.ndarray) -> bool:
    """NaN or +inf anywhere, or no finite maximum."""
    x = np.asarray(x, dtype=np.float32)
    if np.isnan(x).any() or np.isposinf(x).any():
        return True
    return not np.isfinite(np.max(x))


def temp_scale(T) -> np.float32:
    """c = K / T, one float32 division."""
    with np.errstate(over="ignore", divide="ignore"):
        return K_LOG2E_16 / np.float32(T)


def weights(x: np.ndarray, T: float) -> np.ndarray:
    """Integer weights W (int64) of one float32 row at temperature T > 0."""
    Bt = np.array(exp_table(), dtype=np.int64)
    x = np.asarray(x, dtype=np.float32)
    m = np.max(x)
    c = temp_scale(T)
    with np.errstate(invalid="ignore", over="ignore"):
        u = (m - x) * c  # float32 subtraction and product
    W = np.zeros(x.shape, dtype=np.int64)
    ok = u < np.float32(J_MAX)
    j = np.rint(u[ok]).astype(np.int64)
    keep = j < J_MAX
    j = j[keep]
    n, h, r = j >> 16, (j >> 8) & 255, j & 255
    Y = Bt[h] - (((Bt[h] - Bt[h + 1]) * r + 128) >> 8)
    W[np.flatnonzero(ok)[keep]] = (Y + ((1 << n) >> 1)) >> n
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
        elif not (T > 0.0 and np.isfinite(T) and np.isfinite(temp_scale(T))):
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
