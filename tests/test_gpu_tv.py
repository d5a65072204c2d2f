"""GPU parity for the soft accept-rate stage and the config-4 chain.

Tolerances (relative, the stated 1e-5 of fp32 accumulation): the accept rate a
within 1e-5 * a of the fp64 oracle's, and the cumulative product S_k within
1e-5 * k * S_k (each factor adds its own relative error). The errors of
sum min(u, v) computed from base-2 log-partitions are relative to a: the
log-partitions' rounding scales every term alike, and the fp32 sums and
exponentials round relatively; terms below 2^-126 are flushed, at most
V * 2^-126 < 1e-30 in all (the absolute floor below). Downstream of TV the planner is
checked stage-isolated: both sides get the oracle's survivals, rounded to
float32, and must agree bit for bit. In the chained run the GPU planner
consumes the GPU's own survivals. Its integer decisions may then differ from
the oracle's only at a near-tie, which the test verifies from the oracle's
numbers.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.tv import tv_pair
from workloads import f32_to_bf16_bits, make
from _gpu import accept, gather_packed, logits_up, pack, plan, say, tv

pytestmark = pytest.mark.gpu

REL = 1e-5
FLOOR = 1e-30


def _assert_tv(a, S, ref_a, ref_S):
    assert np.all(np.abs(a - ref_a) <= REL * np.abs(ref_a) + FLOOR), \
        np.max(np.abs(a - ref_a) / np.maximum(np.abs(ref_a), FLOOR))
    k = np.arange(1, ref_S.shape[-1] + 1)
    assert np.all(np.abs(S - ref_S) <= REL * k * np.abs(ref_S) + FLOOR)

import json
import os
from pathlib import Path

# the error summary is written only when DSPARK_SUMMARY_DIR names an existing folder
SUMMARY = Path(os.environ.get("DSPARK_SUMMARY_DIR", "/nonexistent")) / "tv_errors.json"


def _record_err(tag, a, S, ref_a, ref_S):
    """Largest absolute and relative errors of a and S against the oracle,
    added to the run's summary (on a GPU run) and printed."""
    tiny = 1e-30
    ea = np.abs(a.astype(np.float64) - ref_a)
    es = np.abs(S.astype(np.float64) - ref_S)
    k = np.arange(1, ref_S.shape[-1] + 1)
    rec = {"pairs": int(a.size), "max_abs_a": float(ea.max()),
           "max_rel_a": float((ea / np.maximum(np.abs(ref_a), tiny)).max()),
           "min_a": float(ref_a.min()), "max_abs_S": float(es.max()),
           "max_rel_S_over_k": float((es / np.maximum(np.abs(ref_S), tiny) / k).max())}
    say(f"{tag}: max |da| {rec['max_abs_a']:.3e}, max |da|/a {rec['max_rel_a']:.3e}, "
        f"max |dS|/(k S) {rec['max_rel_S_over_k']:.3e}")
    if SUMMARY.parent.is_dir():
        data = json.loads(SUMMARY.read_text()) if SUMMARY.exists() else {}
        data[tag] = rec
        SUMMARY.write_text(json.dumps(data, indent=1, sort_keys=True))
    return rec


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(hip):
    return hip


def _rand_logits(rng, shape, sigma, dt):
    x = rng.normal(0, sigma, shape).astype(np.float32)
    return f32_to_bf16_bits(x) if dt == 1 else x


# Row sizes around the kernel's layout limits: pairs of 16-byte vectors up to
# 11 * 1024 stay in registers, up to 4992 more in LDS (16256 vectors: bf16
# V <= 130055 is fully resident), up to 4096 more are read from memory twice
# (20352 vectors: bf16 V <= 162823, fp32 V <= 81411), longer rows take the
# two-pass streaming kernel.
@pytest.mark.parametrize("V,pad,dt", [(257, 0, 1), (257, 7, 1), (1000, 0, 0), (1001, 3, 0),
                                      (4096, 8, 1), (32000, 0, 1), (3, 1, 0),
                                      (90121, 5, 1),    # registers + 1 LDS pair, ragged tail
                                      (130055, 0, 1),   # the largest fully resident bf16 row
                                      (130056, 0, 1),   # one vector more: 1 read twice
                                      (151936, 0, 1),   # 2736 read twice, no tail
                                      (162823, 0, 1),   # the largest such bf16 row
                                      (162824, 0, 1),   # one element more: streaming
                                      (70001, 3, 0),    # fp32, 1244 read twice, ragged tail
                                      (81412, 0, 0),    # fp32, streaming
                                      (262144, 0, 1),   # the largest V the library takes
                                      (262144, 0, 0)])
def test_tv_small(V, pad, dt):
    rng = np.random.default_rng(V * 7 + pad + dt)
    B, G = 3, 4
    epv = 8 if dt == 1 else 4
    ld = V + pad
    ld += (-ld) % epv  # rows must start on 16-byte boundaries
    q = _rand_logits(rng, (B, G, V), 2.0, dt)
    p = _rand_logits(rng, (B, G + 1, V), 2.0, dt)
    q[0, 1] = p[0, 1]  # one identical pair -> a = 1
    nan = np.uint16(0x7FC1) if dt == 1 else np.float32(np.nan)
    qs = np.full((B * G, ld), nan, dtype=q.dtype)
    ps = np.full((B * (G + 1), ld), nan, dtype=p.dtype)  # stride padding: never read
    qs[:, :V] = q.reshape(B * G, V)
    ps[:, :V] = p.reshape(B * (G + 1), V)
    a, S = tv(B, G, V, dt, logits_up(qs, dt), ld, logits_up(ps, dt), ld, G + 1, tag=f"V={V}")
    ref_a, ref_S = oracle.tv_accept(B, G, q, p, "bf16" if dt == 1 else "f32")
    _record_err(f"small V={V} pad={pad} dt={dt}", a, S, ref_a, ref_S)
    _assert_tv(a, S, ref_a, ref_S)
    assert abs(a[0, 1] - 1.0) <= 1e-6
    assert np.all((a >= 0) & (a <= 1))
    # S is the float32 running product of a
    for r in range(B):
        acc = np.float32(1)
        for kk in range(G):
            acc = a[r, kk] if kk == 0 else np.float32(acc * a[r, kk])
            assert S[r, kk] == acc


# More pairs than the chip has CUs: each persistent workgroup then walks
# several pairs, reloading registers and LDS while it finishes the last one.
# Rows with all register slots full (FULL) and shorter ones, ragged tails, an
# LDS part of one pair, and pair counts that do not divide by the CU count.
@pytest.mark.parametrize("V,pad,dt,B,G", [(90121, 5, 1, 37, 9),   # 333 pairs, 1 LDS pair
                                          (130055, 0, 1, 33, 8),  # 264 pairs, full LDS
                                          (151936, 3, 1, 20, 16),  # 320 pairs, 2736 read twice
                                          (98304, 0, 1, 20, 26),  # 520 pairs, 3 per CU at most
                                          (32000, 0, 0, 40, 8),   # fp32, registers only
                                          (45056, 0, 0, 35, 8),   # fp32, exactly 11 * 1024 vectors
                                          (3, 1, 0, 30, 10)])     # tail only
def test_tv_many_pairs(V, pad, dt, B, G):
    rng = np.random.default_rng(V * 13 + B)
    epv = 8 if dt == 1 else 4
    ld = V + pad
    ld += (-ld) % epv
    sig = rng.uniform(0.3, 3.0, (B, 1, 1)).astype(np.float32)
    p32 = rng.normal(0, 2.0, (B, G + 1, V)).astype(np.float32)
    q32 = p32[:, :G] + sig * rng.normal(0, 1.0, (B, G, V)).astype(np.float32)
    q = f32_to_bf16_bits(q32) if dt == 1 else q32
    p = f32_to_bf16_bits(p32) if dt == 1 else p32
    nan = np.uint16(0x7FC1) if dt == 1 else np.float32(np.nan)
    qs = np.full((B * G, ld), nan, dtype=q.dtype)
    ps = np.full((B * (G + 1), ld), nan, dtype=p.dtype)
    qs[:, :V] = q.reshape(B * G, V)
    ps[:, :V] = p.reshape(B * (G + 1), V)
    a, S = tv(B, G, V, dt, logits_up(qs, dt), ld, logits_up(ps, dt), ld, G + 1,
              tag=f"many pairs V={V} pairs={B * G}")
    ref_a, ref_S = oracle.tv_accept(B, G, q, p, "bf16" if dt == 1 else "f32")
    _record_err(f"many pairs V={V} pairs={B * G}", a, S, ref_a, ref_S)
    _assert_tv(a, S, ref_a, ref_S)


# Pass 1 sums each thread's exponentials against the maximum of its first
# vector; a thread whose sums overflow (an element about 2^7 base-2 units
# above that, or a first vector of -inf only) sums again against its exact
# maximum. Spikes far above the rest and -inf blocks take that path.
@pytest.mark.parametrize("V,dt", [(129280, 1), (98304, 1), (32000, 0), (45056, 0),
                                  (151936, 1),   # vectors past the LDS part, read twice
                                  (81408, 0)])   # the same in fp32, the longest such row
def test_tv_overflow_fallback(V, dt):
    rng = np.random.default_rng(V + 5)
    B, G = 6, 4
    epv = 8 if dt == 1 else 4
    p32 = rng.normal(0, 1.0, (B, G + 1, V)).astype(np.float32)
    q32 = p32[:, :G] + rng.normal(0, 0.5, (B, G, V)).astype(np.float32)
    p32[0, 0, V // 2 + 3] = 150.0      # spike in a later vector: overflow
    q32[0, 0, V // 3 + 1] = 149.0
    q32[1, 1, : epv * 1024] = -np.inf   # every thread's first q vector is -inf
    p32[1, 1, : epv * 1024] = -np.inf
    p32[2, 2, :] = -60.0               # flat row, its maximum in thread 0's first
    p32[2, 2, 7] = 200.0               # vector: offsets 375 units apart, no fallback
    q32[3, 0, -1] = 300.0              # the last element (tail or last vector)
    p32[4, 3, V - 3 * epv] = 160.0     # a vector near the end
    q = f32_to_bf16_bits(q32) if dt == 1 else q32
    p = f32_to_bf16_bits(p32) if dt == 1 else p32
    a, S = tv(B, G, V, dt, logits_up(q.reshape(B * G, V), dt), V,
              logits_up(p.reshape(B * (G + 1), V), dt), V, G + 1, tag=f"overflow V={V}")
    ref_a, ref_S = oracle.tv_accept(B, G, q, p, "bf16" if dt == 1 else "f32")
    _record_err(f"overflow V={V} dt={dt}", a, S, ref_a, ref_S)
    assert np.all(np.isfinite(a))
    _assert_tv(a, S, ref_a, ref_S)


def test_tv_closed_forms():
    # uniform q against one spike in p: a = 1/V + (V-1)/(e^L + V - 1)
    V, L = 4096, 6.0
    B, G = 1, 2
    q = np.zeros((B, G, V), np.float32)
    p = np.zeros((B, G + 1, V), np.float32)
    p[0, 0, 17] = L
    p[0, 1, 4000] = L
    q[0, 1, 4000] = L  # identical pair
    a, _ = tv(B, G, V, 0, logits_up(q.reshape(-1, V), 0), V, logits_up(p.reshape(-1, V), 0), V,
              G + 1, tag="closed form")
    expect = 1.0 / V + (V - 1) / (np.exp(L) + V - 1)
    assert abs(a[0, 0] - expect) <= REL * expect
    assert abs(a[0, 1] - 1.0) <= 1e-6


@pytest.fixture(scope="module")
def cfg4():
    say("generating config 4 (q and p logits)")
    w = make(4)
    say("oracle TV over all pairs of config 4")
    a, S = oracle.tv_accept(w.B, w.gamma, w.draft_logits, w.target, "bf16")
    return w, a, S


def _gpu_tv_full(w):
    q_t = logits_up(w.draft_logits.reshape(w.B * w.gamma, w.V), 1)
    p_t = logits_up(w.target.reshape(w.B * (w.gamma + 1), w.V), 1)
    out = tv(w.B, w.gamma, w.V, 1, q_t, w.V, p_t, w.V, w.gamma + 1, tag="cfg4")
    del q_t, p_t
    torch.cuda.empty_cache()
    return out


def test_tv_config4_full(cfg4):
    w, ref_a, ref_S = cfg4
    a, S = _gpu_tv_full(w)
    _record_err("cfg4 (B=256, gamma=16, V=129280 bf16)", a, S, ref_a, ref_S)
    _assert_tv(a, S, ref_a, ref_S)
    assert np.all(S[:, 1:] <= S[:, :-1])


def _plan_survival(w, S32, gpu: bool):
    args = (w.B, w.gamma, oracle.IN_SURVIVAL, S32, None, w.min_len, w.max_len, w.eps, w.b_lo,
            w.b_hi, w.bias, w.alpha, w.theta)
    return plan(*args, tag="cfg4 survival") if gpu else oracle.plan(*args)


def test_config4_planner_stage_isolated(cfg4):
    w, _, ref_S = cfg4
    S32 = ref_S.astype(np.float32)
    got = _plan_survival(w, S32, True)
    ref = _plan_survival(w, S32, False)
    for k in ("verify_lens", "meta", "val", "survival", "sweep"):
        assert np.array_equal(got[k], ref[k], equal_nan=True), k


def test_config4_pack_accept_stage_isolated(cfg4):
    w, _, ref_S = cfg4
    lens = _plan_survival(w, ref_S.astype(np.float32), False)["verify_lens"]
    ref_pack = oracle.pack(w.B, w.gamma, lens, w.anchors, w.drafts, w.tiers, w.prefix_lens)
    got_pack = pack(w.B, w.gamma, lens, w.anchors, w.drafts, w.tiers, w.prefix_lens, tag="cfg4")
    tier = int(ref_pack["meta"][1])
    assert np.array_equal(got_pack["meta"], ref_pack["meta"])
    assert np.array_equal(got_pack["cu_seqlens"], ref_pack["cu_seqlens"])
    assert np.array_equal(got_pack["ids"][:tier], ref_pack["ids"])
    cu = ref_pack["cu_seqlens"]
    rows = gather_packed(w.target, cu, lens, tier)
    got = accept(w.B, w.gamma, w.V, 1, rows, w.V, cu, w.drafts, w.prefix_lens, tag="cfg4")
    ref = oracle.accept(w.B, w.gamma, rows, "bf16", cu, w.drafts, w.prefix_lens)
    total = int(cu[-1])
    assert np.array_equal(got["row_argmax"][:total], ref["row_argmax"])
    for k in ("num_correct", "bonus", "commit", "out_tokens", "prefix_mask", "new_seq", "meta"):
        assert np.array_equal(got[k], ref[k]), k


def test_config4_chained(cfg4):
    w, ref_a, ref_S = cfg4
    a, S = _gpu_tv_full(w)
    got = _plan_survival(w, S, True)
    ref = _plan_survival(w, ref_S.astype(np.float32), False)
    if np.array_equal(got["verify_lens"], ref["verify_lens"]):
        return
    # a disagreement must come from a near-tie the survival error can flip:
    # either two survivals straddling the cut, or two budgets with ratios
    # equal to within the propagated error
    n_diff = int(np.sum(got["verify_lens"] != ref["verify_lens"]))
    say(f"cfg4 chained: {n_diff} requests differ; checking for a near-tie")
    b_star = int(ref["meta"][0])
    s = np.sort(ref["survival"].reshape(-1))[::-1]
    gap = abs(float(s[b_star - 1]) - float(s[b_star])) if 0 < b_star < s.size else np.inf
    sw = ref["sweep"][:, 1]
    gb = int(got["meta"][0])
    ratio_gap = abs(sw[gb] - sw[b_star]) / sw[b_star] if 0 <= gb < sw.size else np.inf
    assert gap <= 2e-5 or ratio_gap <= 2e-5, (gap, ratio_gap)
