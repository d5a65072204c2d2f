"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: integer outputs (verify_lens, b*, cu_seqlens, tier, packed rows, row
argmax, num_correct, bonus, commit, out_tokens, new_seq, prefix_mask) and the
survival bits are bit-exact. tau(b) and ratio(b) are exact too: tau is an
exact integer sum and the ratio one IEEE fp64 division, so the tolerance of
rel 1e-5 is met with zero error.

Stage-isolated runs feed each GPU stage the oracle's upstream outputs, so no
oracle input ever comes from the HIP path. Chained runs go GPU -> GPU -> GPU
and compare the final outputs with the oracle's own chain.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.accept import as_f32_rows
from workloads import make
from _gpu import accept, gather_packed, logits_up, pack, plan, plan_pack, say, tv

pytestmark = pytest.mark.gpu

KIND = {"conf_logits": oracle.IN_CONF_LOGITS, "survival": oracle.IN_SURVIVAL}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(hip):
    return hip


def _eq(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype.kind == "f":
        same = (a.view(np.uint64 if a.itemsize == 8 else np.uint32)
                == b.astype(a.dtype).view(np.uint64 if a.itemsize == 8 else np.uint32))
        nan_both = np.isnan(a) & np.isnan(b)
        bad = ~(same | nan_both)
    else:
        bad = a != b
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} mismatches, first at {idx.tolist()}: "
                             f"gpu={a[tuple(idx[0])]} oracle={b[tuple(idx[0])]}")


def _plan_both(w, b_lo=None, b_hi=None, **over):
    args = dict(B=w.B, gamma=w.gamma, kind=oracle.IN_CONF_LOGITS, conf=w.conf, temps=w.temps,
                min_len=w.min_len, max_len=w.max_len, eps=w.eps,
                b_lo=w.b_lo if b_lo is None else b_lo, b_hi=w.b_hi if b_hi is None else b_hi,
                bias=w.bias, alpha=w.alpha, theta=w.theta)
    args.update(over)
    ref = oracle.plan(*args.values())
    got = plan(*args.values(), tag=f"cfg{w.cfg} seed{w.seed}")
    return got, ref


def _check_plan(got, ref):
    _eq(got["survival"], ref["survival"], "survival")
    _eq(got["verify_lens"], ref["verify_lens"], "verify_lens")
    _eq(got["meta"], ref["meta"], "plan_meta")
    _eq(got["val"], ref["val"], "plan_val")
    if got["sweep"] is not None:
        _eq(got["sweep"], ref["sweep"], "sweep")


# ---------------------------------------------------------------- plan

@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
@pytest.mark.parametrize("seed", [None, 101, 102, 103, 104, 105])
def test_plan_parity(cfg, seed):
    w = make(cfg, seed=seed, logits=False)
    got, ref = _plan_both(w)
    _check_plan(got, ref)


@pytest.mark.parametrize("shift", [-3.0, -1.5, 1.5, 4.0, 6.0])
@pytest.mark.parametrize("cfg", [2, 3])
def test_plan_parity_confidence_shifts(cfg, shift):
    """Low to very high confidence (the confidence-logit mean moved by
    `shift`): survivals spread far below eps, or crowd just under 1, which
    moves the bucket occupancy, the chosen budget and the tier."""
    w = make(cfg, seed=int(1000 + 10 * shift), logits=False, conf_shift=shift)
    got, ref = _plan_both(w)
    _check_plan(got, ref)
    args = (w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len, w.max_len, w.eps,
            w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    gp, gk = plan_pack(*args, w.anchors, w.drafts, w.tiers, w.prefix_lens,
                       tag=f"cfg{cfg} shift {shift}")
    _check_plan_pack(w, args, gp, gk)


def test_plan_pages_examples():
    bias, alpha, theta = np.float32(0), np.zeros(3, np.float32), np.ones(7, np.float32)
    cond = np.array([[0.9, 0.8], [0.6, 0.5]], np.float32)
    for lo, hi in [(2, 2), (0, -1), (0, 1), (3, 4)]:
        args = (2, 2, oracle.IN_COND, cond, None, 1, 3, 0.0, lo, hi, bias, alpha, theta)
        _check_plan(plan(*args, tag=f"pages {lo}-{hi}"), oracle.plan(*args))
    theta = np.full(7, 1e6, np.float32)
    theta[4], theta[5] = 1.0, 1.4
    args = (2, 2, oracle.IN_COND, cond, None, 1, 3, 0.0, 2, 3, bias, alpha, theta)
    got = plan(*args, tag="cost comparison")
    _check_plan(got, oracle.plan(*args))
    assert got["verify_lens"].tolist() == [3, 1]


def test_plan_edge_cases():
    rng = np.random.default_rng(9)
    cases = []
    # ties everywhere, min == max, eps cut, min_len > 1, small budgets
    c = np.full((6, 3), 0.75, np.float32)
    cases.append((6, 3, oracle.IN_COND, c, None, 1, 4, 0.0, 5, 5))
    cases.append((6, 3, oracle.IN_COND, c, None, 2, 2, 0.0, 0, -1))
    cases.append((6, 3, oracle.IN_COND, c, None, 3, 4, 0.3, 0, -1))
    cases.append((6, 3, oracle.IN_COND, c, None, 0, 99, 0.5, 1, 3))
    c2 = np.array([[1.0, 0.5], [0.5, 1.0]], np.float32)
    cases.append((2, 2, oracle.IN_COND, c2, None, 1, 3, 0.0, 2, 2))
    # exactly one eligible candidate, sitting in the last request's slots
    c1 = np.array([[0.01, 0.5], [0.02, 0.5], [0.9, 0.01]], np.float32)
    cases.append((3, 2, oracle.IN_COND, c1, None, 1, 3, 0.5, 0, -1))
    # many identical survivals (crowded buckets -> merge fallback), B not a power of two
    c3 = np.ones((300, 6), np.float32)
    c3[::7] = 0.5
    cases.append((300, 6, oracle.IN_COND, c3, None, 1, 7, 0.0, 0, -1))
    cases.append((300, 6, oracle.IN_COND, c3, None, 2, 5, 0.0, 10, 700))
    s = np.sort(rng.random((40, 5)).astype(np.float32), axis=1)[:, ::-1].copy()
    cases.append((40, 5, oracle.IN_SURVIVAL, s, None, 1, 6, 0.05, 0, -1))
    z = rng.normal(0, 30, (50, 7)).astype(np.float32)  # saturating confidences, subnormal survivals
    cases.append((50, 7, oracle.IN_CONF_LOGITS, z, np.full(7, 1.0, np.float32), 1, 8, 0.0, 0, -1))
    cases.append((1, 64, oracle.IN_CONF_LOGITS, rng.normal(3, 1, (1, 64)).astype(np.float32),
                  rng.uniform(0.5, 2, 64).astype(np.float32), 1, 65, 1e-4, 0, -1))
    cases.append((128, 64, oracle.IN_CONF_LOGITS, rng.normal(2, 2, (128, 64)).astype(np.float32),
                  rng.uniform(0.5, 2, 64).astype(np.float32), 1, 65, 1e-3, 0, -1))
    # gamma 4, 16 and 32 (requests aligned with the waves' lanes); a request
    # whose given survival increases
    s4 = np.sort(rng.random((70, 4)).astype(np.float32), axis=1)[:, ::-1].copy()
    cases.append((70, 4, oracle.IN_SURVIVAL, s4, None, 1, 5, 0.05, 0, -1))
    s4b = s4.copy()
    s4b[33] = [0.5, 0.4, 0.45, 0.1]
    cases.append((70, 4, oracle.IN_SURVIVAL, s4b, None, 1, 5, 0.05, 0, -1))
    c16 = rng.uniform(0.5, 1.0, (40, 16)).astype(np.float32)
    cases.append((40, 16, oracle.IN_COND, c16, None, 1, 17, 1e-3, 0, -1))
    c32 = rng.uniform(0.7, 1.0, (33, 32)).astype(np.float32)
    cases.append((33, 32, oracle.IN_COND, c32, None, 2, 30, 1e-4, 0, -1))
    # 2048 < B * gamma <= 4096: four items per thread
    z12 = rng.normal(1.5, 1.5, (300, 12)).astype(np.float32)
    cases.append((300, 12, oracle.IN_CONF_LOGITS, z12, rng.uniform(0.5, 2, 12).astype(np.float32),
                  1, 13, 1e-4, 0, -1))
    # -0 confidences and survivals rank with +0 (by value, then position, then request)
    cz = np.array([[0.5, -0.0], [0.9, 0.8]], np.float32)
    cases.append((2, 2, oracle.IN_COND, cz, None, 1, 3, 0.0, 0, -1))
    sz = np.array([[0.7, 0.0, 0.0], [0.6, -0.0, -0.0], [-0.0, -0.0, -0.0]], np.float32)
    cases.append((3, 3, oracle.IN_SURVIVAL, sz, None, 1, 4, 0.0, 0, -1))
    cases.append((3, 3, oracle.IN_SURVIVAL, sz, None, 1, 4, -1.0, 4, 7))
    for i, (B, G, kind, conf, temps, mn, mx, eps, lo, hi) in enumerate(cases):
        alpha = (np.arange(B + 1) * 0.01).astype(np.float32)
        theta = (0.3 + 0.01 * np.arange(B * (G + 1) + 1)).astype(np.float32)
        args = (B, G, kind, conf, temps, mn, mx, eps, lo, hi, np.float32(0.5), alpha, theta)
        _check_plan(plan(*args, tag=f"edge{i}"), oracle.plan(*args))


def test_plan_empty_batch():
    alpha, theta = np.zeros(1, np.float32), np.ones(1, np.float32)
    args = (0, 4, oracle.IN_COND, np.zeros((0, 4), np.float32), None, 1, 5, 0.0, 0, -1,
            np.float32(0.5), alpha, theta)
    got = plan(*args, tag="B=0")
    ref = oracle.plan(*args)
    _eq(got["meta"], ref["meta"], "meta")
    _eq(got["val"], ref["val"], "val")


def test_plan_bad_data_fallback():
    w = make(1, logits=False)
    theta = w.theta.copy()
    theta[w.B + 5] = -10.0
    got, ref = _plan_both(w, theta=theta)
    _check_plan(got, ref)
    assert got["meta"][2] == oracle.DATA_BAD_COST
    temps = w.temps.copy()
    temps[3] = 0.0
    got, ref = _plan_both(w, temps=temps)
    _check_plan(got, ref)
    assert got["meta"][2] == oracle.DATA_BAD_CONF
    conf = w.conf.copy()
    conf[2, 2] = np.nan
    got, ref = _plan_both(w, conf=conf)
    _check_plan(got, ref)


def test_sigmoid_bits_over_many_inputs():
    """Survivals with gamma = 1 and T = 1 are the sigmoid itself: compare bits
    over 2**21 inputs spanning the whole range (plus ones that take the
    device's exact path, found with the host build of the same code)."""
    from dspark_verify_scheduling_amd import _lib

    rng = np.random.default_rng(11)
    x = np.concatenate([rng.normal(0, 6, 1 << 20), rng.uniform(-110, 20, 1 << 20)]).astype(np.float32)
    hc = _lib.hostcheck()
    probe = rng.uniform(-40, 18, 1 << 22).astype(np.float32)
    y = np.empty_like(probe)
    slow = np.zeros(probe.shape, np.uint8)
    hc.dspark_hostcheck_sigmoid(probe.ctypes.data, y.ctypes.data, slow.ctypes.data, probe.size, 0)
    x = np.concatenate([x, probe[slow.astype(bool)]])
    say(f"sigmoid bits: {x.size} inputs, {int(slow.sum())} on the exact path")
    B = 8192
    alpha, theta = np.zeros(B + 1, np.float32), np.ones(2 * B + 1, np.float32)
    ref = oracle.sigmoid32(x)
    for i in range(0, x.size, B):
        chunk = x[i:i + B]
        n = chunk.size
        got = plan(n, 1, oracle.IN_CONF_LOGITS, chunk.reshape(n, 1), np.ones(1, np.float32), 1, 1,
                   0.0, 0, -1, 0.0, alpha[: n + 1], theta[: 2 * n + 1], sweep=False,
                   tag=f"sigmoid {i}")
        _eq(got["survival"].reshape(-1), ref[i:i + n], f"sigmoid chunk {i}")


# ---------------------------------------------------------------- pack

@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
@pytest.mark.parametrize("seed", [None, 201])
def test_pack_parity(cfg, seed):
    w = make(cfg, seed=seed, logits=False)
    ref_plan = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                           w.max_len, w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    lens = ref_plan["verify_lens"]
    ref = oracle.pack(w.B, w.gamma, lens, w.anchors, w.drafts, w.tiers, w.prefix_lens)
    got = pack(w.B, w.gamma, lens, w.anchors, w.drafts, w.tiers, w.prefix_lens, tag=f"cfg{cfg}")
    tier = int(ref["meta"][1])
    _eq(got["meta"], ref["meta"], "pack_meta")
    _eq(got["cu_seqlens"], ref["cu_seqlens"], "cu_seqlens")
    for k in ("ids", "req", "pos"):
        _eq(got[k][:tier], ref[k], k)
        assert np.all(got[k][tier:] == -7), f"{k} written past the tier"


def test_pack_edge_cases():
    rng = np.random.default_rng(3)
    B, G = 37, 5
    anchors = rng.integers(0, 1000, B).astype(np.int32)
    drafts = rng.integers(0, 1000, (B, G)).astype(np.int32)
    tiers = [40, 64, 128, 222]
    for lens, prefix, req, pos in [
        (np.ones(B, np.int32), None, True, True),
        (np.full(B, G + 1, np.int32), rng.integers(0, 99, B), True, False),
        (rng.integers(1, G + 2, B).astype(np.int32), rng.integers(0, 99, B), False, True),
        (rng.integers(-2, G + 4, B).astype(np.int32), None, True, True),  # malformed -> clamped
    ]:
        ref = oracle.pack(B, G, lens, anchors, drafts, tiers, prefix)
        got = pack(B, G, lens, anchors, drafts, tiers, prefix, req=req, pos=pos, tag="edge")
        tier = int(ref["meta"][1])
        _eq(got["meta"], ref["meta"], "meta")
        _eq(got["cu_seqlens"], ref["cu_seqlens"], "cu")
        _eq(got["ids"][:tier], ref["ids"], "ids")
        if req:
            _eq(got["req"][:tier], ref["req"], "req")
        if pos:
            _eq(got["pos"][:tier], ref["pos"], "pos")
    got = pack(0, 3, np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros((0, 3), np.int32),
               [4], tag="B=0")
    assert got["meta"].tolist() == [0, 4, 0] and got["cu_seqlens"].tolist() == [0]


# ---------------------------------------------------------------- fused plan + pack

def _check_plan_pack(w, args, got_plan, got_pack):
    ref_plan = oracle.plan(*args)
    _check_plan(got_plan, ref_plan)
    ref_pack = oracle.pack(w.B, w.gamma, ref_plan["verify_lens"], w.anchors, w.drafts, w.tiers,
                           w.prefix_lens)
    tier = int(ref_pack["meta"][1])
    _eq(got_pack["meta"], ref_pack["meta"], "pack_meta")
    _eq(got_pack["cu_seqlens"], ref_pack["cu_seqlens"], "cu_seqlens")
    for k in ("ids", "req", "pos"):
        _eq(got_pack[k][:tier], ref_pack[k], k)
        assert np.all(got_pack[k][tier:] == -7), f"{k} written past the tier"


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
@pytest.mark.parametrize("seed", [None, 401, 402])
def test_plan_pack_parity(cfg, seed):
    w = make(cfg, seed=seed, logits=False)
    args = (w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len, w.max_len, w.eps,
            w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    gp, gk = plan_pack(*args, w.anchors, w.drafts, w.tiers, w.prefix_lens, tag=f"cfg{cfg}")
    _check_plan_pack(w, args, gp, gk)


def test_plan_pack_fallback_and_limits():
    w = make(1, logits=False)
    theta = w.theta.copy()
    theta[w.B + 2] = -1.0  # bad cost: static window, packed
    args = (w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len, w.max_len, w.eps,
            w.b_lo, w.b_hi, w.bias, w.alpha, theta)
    gp, gk = plan_pack(*args, w.anchors, w.drafts, w.tiers, w.prefix_lens, tag="bad cost")
    _check_plan_pack(w, args, gp, gk)
    assert gk["meta"][0] == w.B * (w.gamma + 1)
    conf = w.conf.copy()
    conf[0, 0] = np.nan  # bad confidence
    args = args[:3] + (conf,) + args[4:12] + (w.theta,)
    gp, gk = plan_pack(*args, w.anchors, w.drafts, w.tiers, w.prefix_lens, tag="bad conf")
    _check_plan_pack(w, args, gp, gk)
    # largest candidate count: B * gamma = 8192, cfg-3-like inputs
    rng = np.random.default_rng(17)
    B, G = 1024, 8
    conf = (rng.normal(1.2, 1.2, (B, G)) - 0.3 * np.arange(1, G + 1)).astype(np.float32)
    temps = rng.uniform(0.7, 2.0, G).astype(np.float32)
    alpha = (0.005 * np.arange(B + 1)).astype(np.float32)
    theta = (0.5 + 0.002 * np.arange(B * (G + 1) + 1)).astype(np.float32)
    anchors = rng.integers(0, 1000, B).astype(np.int32)
    drafts = rng.integers(0, 1000, (B, G)).astype(np.int32)
    tiers = np.array([1024, 2048, 4096, 8192, 9216], np.int32)

    class W:
        pass

    wl = W()
    wl.B, wl.gamma, wl.anchors, wl.drafts, wl.tiers, wl.prefix_lens = B, G, anchors, drafts, tiers, None
    args = (B, G, oracle.IN_CONF_LOGITS, conf, temps, 1, G + 1, 1e-3, 0, -1, np.float32(0.5),
            alpha, theta)
    gp, gk = plan_pack(*args, anchors, drafts, tiers, None, tag="B*gamma=8192")
    _check_plan_pack(wl, args, gp, gk)


# ---------------------------------------------------------------- accept

_WL = {}


def _workload(cfg, seed=None):
    key = (cfg, seed)
    if key not in _WL:
        say(f"generating workload cfg{cfg} seed{seed}")
        _WL.clear()
        _WL[key] = make(cfg, seed=seed)
    return _WL[key]


def _accept_both(w, lens, tag):
    ref_pack = oracle.pack(w.B, w.gamma, lens, w.anchors, w.drafts, w.tiers, w.prefix_lens)
    cu = ref_pack["cu_seqlens"]
    tier = int(ref_pack["meta"][1])
    rows = gather_packed(w.target, cu, lens, tier)
    dt = 1 if w.dtype == "bf16" else 0
    got = accept(w.B, w.gamma, w.V, dt, rows, w.V, cu, w.drafts, w.prefix_lens, tag=tag)
    ref = oracle.accept(w.B, w.gamma, rows, w.dtype, cu, w.drafts, w.prefix_lens)
    return got, ref, int(cu[-1])


def _check_accept(got, ref, total):
    _eq(got["row_argmax"][:total], ref["row_argmax"], "row_argmax")
    for k in ("num_correct", "bonus", "commit", "out_tokens", "prefix_mask", "meta"):
        _eq(got[k], ref[k], k)
    if got["new_seq"] is not None:
        _eq(got["new_seq"], ref["new_seq"], "new_seq")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_accept_parity_planned(cfg):
    w = _workload(cfg)
    ref_plan = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                           w.max_len, w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    got, ref, total = _accept_both(w, ref_plan["verify_lens"], f"cfg{cfg} planned")
    _check_accept(got, ref, total)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_accept_parity_static(cfg):
    """verify_lens = gamma + 1 for every request (static mode): the packed
    layout equals the strided one."""
    w = _workload(cfg)
    lens = np.full(w.B, w.gamma + 1, np.int32)
    got, ref, total = _accept_both(w, lens, f"cfg{cfg} static")
    _check_accept(got, ref, total)
    # static mode against plain leading-match counting on the strided rows
    am = ref["row_argmax"].reshape(w.B, w.gamma + 1)
    for r in range(min(w.B, 64)):
        n = 0
        while n < w.gamma and w.drafts[r, n] == am[r, n]:
            n += 1
        assert got["num_correct"][r] == n


@pytest.mark.parametrize("seed", [301, 302])
def test_accept_parity_other_seeds(seed):
    w = _workload(2, seed)
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, w.gamma + 2, w.B).astype(np.int32)
    got, ref, total = _accept_both(w, lens, f"cfg2 seed{seed} random lens")
    _check_accept(got, ref, total)


def _edge_rows(rng, n, V, dt):
    """Rows exercising ties, NaN, signed zeros, infinities, constant rows."""
    x = rng.normal(0, 3, (n, V)).astype(np.float32)
    kinds = []
    for i in range(n):
        k = i % 8
        kinds.append(k)
        if k == 1 and V >= 2:  # exact tie between two far-apart ids
            a, b = sorted(rng.choice(V, 2, replace=False))
            x[i, a] = x[i, b] = 50.0
        elif k == 2:  # NaN somewhere: the first NaN wins
            x[i, rng.integers(0, V)] = np.nan
            x[i, rng.integers(0, V)] = np.nan
        elif k == 3:  # all zeros with signs mixed
            x[i] = np.where(rng.random(V) < 0.5, -0.0, 0.0)
        elif k == 4:  # all -inf
            x[i] = -np.inf
        elif k == 5:  # constant row
            x[i] = 1.25
        elif k == 6:  # +inf twice
            x[i, rng.integers(0, V, 2)] = np.inf
        elif k == 7:  # maximum in the last element (tail)
            x[i, V - 1] = 99.0
    if dt == 1:
        from workloads import f32_to_bf16_bits

        bits = f32_to_bf16_bits(np.nan_to_num(x, nan=0.0, posinf=np.inf, neginf=-np.inf))
        bits[np.isnan(x)] = 0x7FC1
        # a negative NaN in some rows
        for i in range(n):
            if kinds[i] == 2 and i % 16 == 2:
                bits[i, 0] = 0xFFC3
        return bits
    return x


@pytest.mark.parametrize("V,ld,dt", [
    (1000, 1000, 0), (1000, 1008, 1), (1001, 1008, 1), (1001, 1004, 0), (7, 8, 1), (1, 4, 0),
    (16, 16, 1), (129280, 129280, 1), (32000, 32004, 0), (262144, 262144, 1),
])
def test_accept_edge_rows(V, ld, dt):
    rng = np.random.default_rng(V + ld + dt)
    B, G = 9, 3
    rows_n = B * (G + 1)
    data = _edge_rows(rng, rows_n, V, dt)
    rows = np.empty((rows_n + 5, ld), dtype=data.dtype)
    rows[:] = np.uint16(0x7F80) if dt == 1 else np.float32(np.inf)  # stride padding: +inf
    rows[:rows_n, :V] = data
    lens = rng.integers(1, G + 2, B).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    am_true = oracle.row_argmax(as_f32_rows(rows[:, :V], "bf16" if dt else "f32"))
    drafts = np.where(rng.random((B, G)) < 0.6,
                      am_true[np.minimum(cu[:-1, None] + np.arange(G), rows_n - 1)],
                      rng.integers(0, V, (B, G))).astype(np.int32)
    prefix = rng.integers(0, 500, B).astype(np.int32)
    got = accept(B, G, V, dt, rows, ld, cu, drafts, prefix, tag=f"edge V={V}")
    ref = oracle.accept(B, G, rows[:, :V], "bf16" if dt else "f32", cu, drafts, prefix,
                        max_rows=rows.shape[0])
    _check_accept(got, ref, int(cu[-1]))


@pytest.mark.parametrize("dt", [0, 1])
def test_accept_gamma_64(dt):
    """gamma = 64, the largest: a request of gamma + 1 = 65 rows reads one row
    more than a wave has lanes, and the match count runs over 64 drafts."""
    rng = np.random.default_rng(64 + dt)
    B, G, V = 5, 64, 2048
    lens = np.array([65, 65, 1, 30, 64], np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = rng.normal(0, 2, (int(cu[-1]) + 3, V)).astype(np.float32)
    rows = x if dt == 0 else (x.view(np.uint32) >> 16).astype(np.uint16)
    am = oracle.row_argmax(as_f32_rows(rows, "bf16" if dt else "f32"))
    # draft k matches the prediction of row k - 1 up to a chosen first miss
    first_miss = [G, G - 1, 0, 10, 63]  # G: every draft matches
    drafts = np.empty((B, G), np.int32)
    for r in range(B):
        for k in range(G):
            row = min(int(cu[r]) + k, x.shape[0] - 1)
            drafts[r, k] = am[row] if k < first_miss[r] else (am[row] + 1) % V
    prefix = rng.integers(0, 1000, B).astype(np.int32)
    got = accept(B, G, V, dt, rows, V, cu, drafts, prefix, tag=f"gamma=64 dt={dt}")
    ref = oracle.accept(B, G, rows, "bf16" if dt else "f32", cu, drafts, prefix,
                        max_rows=rows.shape[0])
    assert ref["num_correct"].tolist() == [64, 63, 0, 10, 63]
    _check_accept(got, ref, int(cu[-1]))


def test_accept_malformed_layouts_and_reuse():
    rng = np.random.default_rng(5)
    B, G, V = 4, 3, 4096
    rows = rng.normal(size=(12, V)).astype(np.float32)
    drafts = rng.integers(0, V, (B, G)).astype(np.int32)
    prefix = np.arange(B, dtype=np.int32)
    import dspark_verify_scheduling_amd as dv

    outs = dv.alloc_accept_outputs(B, G, 12, V, 0, "cuda", new_seq=True, mask=True)
    for cu in ([0, 2, 2, 5, 7], [0, 3, 5, 9, 14], [0, 5, 6, 7, 8], [0, 1, 2, 3, 4], [0, 4, 8, 12, 16],
               [3, 4, 5, 6, 7]):
        cu = np.asarray(cu, np.int32)
        got = accept(B, G, V, 0, rows, V, cu, drafts, prefix, outs=outs, tag=f"cu={cu.tolist()}")
        ref = oracle.accept(B, G, rows, "f32", cu, drafts, prefix, max_rows=12)
        _check_accept(got, ref, min(max(int(cu[-1]), 0), 12))


def test_accept_determinism():
    w = _workload(1)
    lens = np.full(w.B, w.gamma + 1, np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rows = gather_packed(w.target, cu, lens, int(cu[-1]))
    t = logits_up(rows, 0)
    first = accept(w.B, w.gamma, w.V, 0, None, w.V, cu, w.drafts, w.prefix_lens,
                   max_rows=rows.shape[0], logits_t=t, tag="determinism 0")
    for i in range(1, 20):
        again = accept(w.B, w.gamma, w.V, 0, None, w.V, cu, w.drafts, w.prefix_lens,
                       max_rows=rows.shape[0], logits_t=t, tag=f"determinism {i}")
        for k in ("row_argmax", "num_correct", "bonus", "out_tokens"):
            _eq(again[k], first[k], k)


# ---------------------------------------------------------------- chained

@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_chained_plan_pack_accept(cfg):
    import dspark_verify_scheduling_amd as dv

    w = _workload(cfg)
    dt = 1 if w.dtype == "bf16" else 0
    # GPU chain
    g_plan = plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len, w.max_len,
                  w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta, tag=f"chain cfg{cfg}")
    g_pack = pack(w.B, w.gamma, g_plan["verify_lens"], w.anchors, w.drafts, w.tiers,
                  w.prefix_lens, tag=f"chain cfg{cfg}")
    # the target forward's stand-in: gather strided rows on the device by packed request/row
    strided = logits_up(w.target.reshape(w.rows_strided, w.V), dt)
    req = torch.from_numpy(g_pack["req"]).cuda().long()
    cu_t = torch.from_numpy(g_pack["cu_seqlens"]).cuda().long()
    tier = int(g_pack["meta"][1])
    idx = torch.arange(tier, device="cuda")
    valid = req[:tier] >= 0
    src = torch.where(valid, req[:tier] * (w.gamma + 1) + (idx - cu_t[req[:tier].clamp(min=0)]),
                      torch.zeros_like(idx))
    packed_t = strided.index_select(0, src).contiguous()
    del strided
    g_acc = accept(w.B, w.gamma, w.V, dt, None, w.V, g_pack["cu_seqlens"], w.drafts,
                   w.prefix_lens, max_rows=tier, logits_t=packed_t, tag=f"chain cfg{cfg}")
    # oracle chain
    o_plan = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                         w.max_len, w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    o_pack = oracle.pack(w.B, w.gamma, o_plan["verify_lens"], w.anchors, w.drafts, w.tiers,
                         w.prefix_lens)
    o_rows = gather_packed(w.target, o_pack["cu_seqlens"], o_plan["verify_lens"],
                           int(o_pack["meta"][1]))
    o_acc = oracle.accept(w.B, w.gamma, o_rows, w.dtype, o_pack["cu_seqlens"], w.drafts,
                          w.prefix_lens)
    _check_plan(g_plan, o_plan)
    _eq(g_pack["cu_seqlens"], o_pack["cu_seqlens"], "cu")
    _eq(g_pack["meta"], o_pack["meta"], "pack meta")
    _check_accept(g_acc, o_acc, int(o_pack["meta"][0]))
    # Σ commit = B + Σ correct
    assert int(g_acc["commit"].sum()) == w.B + int(g_acc["num_correct"].sum())


def test_graph_replay_matches_eager():
    """plan + pack + accept captured in one HIP graph; every replay, with eager
    work in between, matches the eager result."""
    import dspark_verify_scheduling_amd as dv

    w = _workload(1)
    dt = 0
    B, G = w.B, w.gamma
    cap = int(w.tiers[-1])
    lens_ref = oracle.plan(B, G, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len, w.max_len,
                           w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)["verify_lens"]
    cu_ref = np.concatenate([[0], np.cumsum(lens_ref)])
    rows = gather_packed(w.target, cu_ref, lens_ref, cap)
    conf_t = torch.from_numpy(w.conf).cuda()
    temps_t = torch.from_numpy(w.temps).cuda()
    alpha_t = torch.from_numpy(w.alpha).cuda()
    theta_t = torch.from_numpy(w.theta).cuda()
    anchors_t = torch.from_numpy(w.anchors).cuda()
    drafts_t = torch.from_numpy(w.drafts).cuda()
    prefix_t = torch.from_numpy(w.prefix_lens).cuda()
    logits_t = logits_up(rows, dt)
    po = dv.alloc_plan_outputs(B, G, "cuda", survival=False)
    ko = dv.alloc_pack_outputs(B, cap, "cuda")
    ao = dv.alloc_accept_outputs(B, G, cap, w.V, dt, "cuda")

    def step():
        dv.dspark_plan(B, G, dv.IN_CONF_LOGITS, conf_t, temps_t, w.min_len, w.max_len, w.eps,
                       w.b_lo, w.b_hi, float(w.bias), alpha_t, theta_t, po)
        dv.dspark_pack(B, G, po.verify_lens, anchors_t, drafts_t, list(w.tiers), prefix_t, ko)
        dv.dspark_accept(B, G, w.V, dt, logits_t, w.V, cap, ko.cu_seqlens, drafts_t, prefix_t, ao)

    say("graph: eager step")
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (po.verify_lens, ko.cu_seqlens, ao.row_argmax[: int(cu_ref[-1])],
                                 ao.num_correct, ao.bonus, ao.out_tokens, ao.commit_lens)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g):
        step()
    for i in range(5):
        say(f"graph: replay {i}")
        for t in (po.verify_lens, ko.cu_seqlens, ao.num_correct, ao.out_tokens):
            t.fill_(-3)
        g.replay()
        torch.cuda.synchronize()
        now = [po.verify_lens, ko.cu_seqlens, ao.row_argmax[: int(cu_ref[-1])], ao.num_correct,
               ao.bonus, ao.out_tokens, ao.commit_lens]
        for a, b in zip(now, eager):
            assert torch.equal(a, b), f"replay {i} differs"
        step()  # eager work between replays
        torch.cuda.synchronize()
