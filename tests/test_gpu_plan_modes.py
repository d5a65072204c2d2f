"""GPU parity of dspark_plan_pack_ex (1D SPS cost mode, graph-tier
alignment) against the CPU oracle, through the C ABI.

Bar: as for the planner: verify_lens, plan_meta, survival bits, tau and the
objective (sweep and plan_val) bit-exact, and the packed layout bit-exact.
"""

import numpy as np
import pytest

import oracle
from workloads import make
from _gpu import plan_pack_ex, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(hip):
    return hip


def _eq(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype.kind == "f":
        bits = np.uint64 if a.itemsize == 8 else np.uint32
        bad = ~((a.view(bits) == b.astype(a.dtype).view(bits)) | (np.isnan(a) & np.isnan(b)))
    else:
        bad = a != b
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} mismatches, first at {idx.tolist()}: "
                             f"gpu={a[tuple(idx[0])]} oracle={b[tuple(idx[0])]}")


def _sps_table(w, rng, n_random=12, cliff=True, first_above_min=False):
    """Probe totals at the tiers and some random totals; steps/s from the
    workload's additive cost (1000 / T ms), with a cliff past one tier."""
    lmin = max(1, w.min_len)
    m_lo, m_hi = w.B * lmin, w.B * (w.gamma + 1)
    pts = set(int(t) for t in w.tiers if t <= m_hi)
    pts |= set(rng.integers(m_lo, m_hi + 1, size=n_random).tolist())
    pts.add(m_lo + 3 if first_above_min else m_lo)
    pts = np.array(sorted(p for p in pts if (p > m_lo + 2 or not first_above_min)), np.int32)
    T = np.float64(w.bias) + np.float64(w.alpha[w.B]) + w.theta[pts].astype(np.float64)
    sps = 1000.0 / T
    if cliff and len(pts) > 2:
        sps[len(pts) // 2:] *= 0.6
    return pts, sps.astype(np.float32)


def _both(w, conf=None, kind=oracle.IN_CONF_LOGITS, temps="w", cost_mode=0, sps_m=None,
          sps=None, align=False, tag=""):
    conf = w.conf if conf is None else conf
    temps = w.temps if temps == "w" else temps
    args = (w.B, w.gamma, kind, conf, temps, w.min_len, w.max_len, w.eps, w.b_lo, w.b_hi,
            w.bias, w.alpha, w.theta)
    gp, gk = plan_pack_ex(*args, w.anchors, w.drafts, w.tiers, w.prefix_lens,
                          cost_mode=cost_mode, sps_m=sps_m, sps=sps, align=align, tag=tag)
    rp = oracle.plan(*args, cost_mode=cost_mode, sps_m=sps_m, sps=sps,
                     align_tiers=w.tiers if align else None)
    for k in ("survival", "verify_lens", "meta", "val", "sweep"):
        _eq(gp[k], rp[k], k)
    rk = oracle.pack(w.B, w.gamma, rp["verify_lens"], w.anchors, w.drafts, w.tiers, w.prefix_lens)
    tier = int(rk["meta"][1])
    _eq(gk["meta"], rk["meta"], "pack_meta")
    _eq(gk["cu_seqlens"], rk["cu_seqlens"], "cu_seqlens")
    for k in ("ids", "req", "pos"):
        _eq(gk[k][:tier], rk[k], k)
        assert np.all(gk[k][tier:] == -7), f"{k} written past the tier"
    return gp, rp


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
@pytest.mark.parametrize("seed", [None, 501])
def test_sps1d_parity(cfg, seed):
    w = make(cfg, seed=seed, logits=False)
    rng = np.random.default_rng(cfg * 10 + (seed or 0))
    sps_m, sps = _sps_table(w, rng)
    gp, rp = _both(w, cost_mode=oracle.COST_SPS1D, sps_m=sps_m, sps=sps, tag=f"cfg{cfg} sps1d")
    say(f"cfg{cfg}: SPS1D b* = {rp['meta'][0]} of {rp['meta'][1]} candidates")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_alignment_parity(cfg):
    w = make(cfg, logits=False)
    gp, rp = _both(w, align=True, tag=f"cfg{cfg} aligned")
    assert rp["meta"][3] >= w.B * w.min_len + rp["meta"][0]
    say(f"cfg{cfg}: aligned b* = {rp['meta'][0]} -> executed total {rp['meta'][3]}")


def test_sps1d_with_alignment_and_edge_tables():
    w = make(3, logits=False)
    rng = np.random.default_rng(9)
    sps_m, sps = _sps_table(w, rng)
    _both(w, cost_mode=oracle.COST_SPS1D, sps_m=sps_m, sps=sps, align=True, tag="sps1d aligned")
    # a single probe; a first probe above the smallest total; the most probes
    _both(w, cost_mode=oracle.COST_SPS1D, sps_m=np.array([w.B + 100], np.int32),
          sps=np.array([50.0], np.float32), tag="one probe")
    m2, s2 = _sps_table(w, rng, first_above_min=True)
    assert m2[0] > w.B * w.min_len
    _both(w, cost_mode=oracle.COST_SPS1D, sps_m=m2, sps=s2, tag="first probe above min")
    m3 = np.arange(w.B, w.B + 512, dtype=np.int32) * 4 // 1
    m3 = np.unique(np.minimum(m3, w.B * (w.gamma + 1) + 600))[:512].astype(np.int32)
    s3 = (1000.0 / (1.0 + 0.01 * np.arange(m3.size))).astype(np.float32)
    _both(w, cost_mode=oracle.COST_SPS1D, sps_m=m3, sps=s3, tag=f"{m3.size} probes")


def test_sps1d_bad_tables_fall_back():
    w = make(1, logits=False)
    for m, v, what in (([20, 20, 40], [3, 2, 1], "repeated probe"),
                       ([30, 10], [1, 1], "descending probes"),
                       ([8, 40], [100.0, 0.0], "zero SPS"),
                       ([8, 40], [100.0, np.inf], "infinite SPS")):
        gp, rp = _both(w, cost_mode=oracle.COST_SPS1D, sps_m=np.array(m, np.int32),
                       sps=np.array(v, np.float32), tag=what)
        assert rp["meta"][2] == oracle.DATA_BAD_COST, what
    # a bad confidence wins over a bad table, as in the oracle
    conf = w.conf.copy()
    conf[1, 1] = np.nan
    gp, rp = _both(w, conf=conf, cost_mode=oracle.COST_SPS1D, sps_m=np.array([30, 10], np.int32),
                   sps=np.array([1, 1], np.float32), tag="bad conf and bad table")
    assert rp["meta"][2] == oracle.DATA_BAD_CONF


def test_largest_problem_sps1d_aligned():
    """B * gamma = 8192 candidates with the full probe table and alignment."""
    w = make(3, logits=False)
    B, G = 1024, 8
    rng = np.random.default_rng(11)
    conf = (rng.normal(1.2, 1.2, size=(B, G)) - 0.3 * np.arange(1, G + 1)).astype(np.float32)
    tiers = [1024, 2048, 4096, 8192, 9216]
    m = np.unique(rng.integers(B, B * (G + 1) + 1, size=600)).astype(np.int32)[:512]
    s = np.sort(rng.uniform(10.0, 200.0, size=m.size))[::-1].astype(np.float32)
    alpha = np.zeros(B + 1, np.float32)
    theta = np.ones(B * (G + 1) + 1, np.float32)
    anchors = rng.integers(0, 1000, B).astype(np.int32)
    drafts = rng.integers(0, 1000, (B, G)).astype(np.int32)
    prefix = rng.integers(0, 100, B).astype(np.int32)
    args = (B, G, oracle.IN_CONF_LOGITS, conf, w.temps, 1, G + 1, 1e-3, 0, -1, 0.5, alpha, theta)
    gp, gk = plan_pack_ex(*args, anchors, drafts, tiers, prefix, cost_mode=oracle.COST_SPS1D,
                          sps_m=m, sps=s, align=True, tag="B*gamma=8192")
    rp = oracle.plan(*args, cost_mode=oracle.COST_SPS1D, sps_m=m, sps=s, align_tiers=tiers)
    for k in ("survival", "verify_lens", "meta", "val", "sweep"):
        _eq(gp[k], rp[k], k)
    rk = oracle.pack(B, G, rp["verify_lens"], anchors, drafts, tiers, prefix)
    _eq(gk["meta"], rk["meta"], "pack_meta")
    tier = int(rk["meta"][1])
    for k in ("ids", "req", "pos"):
        _eq(gk[k][:tier], rk[k], k)
