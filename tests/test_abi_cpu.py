"""C-ABI checks that need no GPU.

* libdspark.so loads and exports every function include/dspark.h declares.
* Argument errors are caught on the host, before any launch, with the
  documented status codes. No call here reaches a kernel launch.
* The device sigmoid, compiled for the host, equals the oracle's correctly
  rounded sigmoid bit for bit on both of its paths (the fp64 fast path and
  the double-double path that real inputs reach about once per million).
"""

import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

from dspark_verify_scheduling_amd import _lib
from oracle.sigmoid import nearest_f32, sigmoid32, sigmoid_decimal

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "dspark.h"

NULL = None
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def _declared():
    text = HEADER.read_text(encoding="utf-8")
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("dspark_plan", "dspark_pack", "dspark_plan_pack", "dspark_accept", "dspark_tv_accept",
              "dspark_accept_workspace_size", "dspark_status_str", "dspark_last_error",
              "dspark_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_lib.SIGNATURES) == set(_declared())
    assert lib.dspark_version() >> 16 == 1


def test_status_strings():
    assert _lib.status_str(0) == "DSPARK_OK"
    assert _lib.status_str(2) == "DSPARK_E_UNSUPPORTED"


def _plan(**kw):
    a = dict(B=4, gamma=4, kind=0, conf=FAKE, temp=FAKE, mn=1, mx=5, eps=1e-3, lo=0, hi=-1,
             bias=0.5, alpha=FAKE, alen=5, theta=FAKE, tlen=21, lens=FAKE, meta=FAKE, val=FAKE,
             surv=NULL, sweep=NULL, stream=NULL)
    a.update(kw)
    return _lib.lib().dspark_plan(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), _lib.E_INVALID),
    (dict(gamma=0), _lib.E_INVALID),
    (dict(gamma=65), _lib.E_INVALID),
    (dict(kind=7), _lib.E_INVALID),
    (dict(B=1025, gamma=8), _lib.E_UNSUPPORTED),
    (dict(B=8193, gamma=1, alen=9000, tlen=20000), _lib.E_UNSUPPORTED),
    (dict(conf=NULL), _lib.E_INVALID),
    (dict(temp=NULL), _lib.E_INVALID),
    (dict(alpha=NULL), _lib.E_INVALID),
    (dict(lens=NULL), _lib.E_INVALID),
    (dict(lo=-1), _lib.E_INVALID),
    (dict(lo=3, hi=2), _lib.E_INVALID),
    (dict(eps=float("nan")), _lib.E_INVALID),
    (dict(alen=4), _lib.E_INVALID),
    (dict(tlen=20), _lib.E_INVALID),  # needs > B * L_max = 20
])
def test_plan_argument_errors(kw, code):
    assert _plan(**kw) == code
    assert _lib.last_error() != ""


def test_plan_pack_argument_errors():
    tiers = (ctypes.c_int32 * 2)(8, 20)
    base = dict(B=4, gamma=4, kind=0, conf=FAKE, temp=FAKE, mn=1, mx=5, eps=1e-3, lo=0, hi=-1,
                bias=0.5, alpha=FAKE, alen=5, theta=FAKE, tlen=21, lens=FAKE, meta=FAKE, val=FAKE,
                surv=NULL, sweep=NULL, anchors=FAKE, drafts=FAKE,
                tiers=ctypes.cast(tiers, ctypes.c_void_p), ntiers=2, prefix=NULL, cu=FAKE,
                ids=FAKE, req=NULL, pos=NULL, pmeta=FAKE, stream=NULL)

    def run(**kw):
        d = dict(base)
        d.update(kw)
        return _lib.lib().dspark_plan_pack(*d.values())

    assert run(gamma=0) == _lib.E_INVALID  # plan rule
    assert run(tlen=20) == _lib.E_INVALID  # plan rule
    assert run(ntiers=1) == _lib.E_INVALID  # last tier 8 < B * (gamma + 1) = 20
    assert run(anchors=NULL) == _lib.E_INVALID  # pack rule
    assert run(cu=NULL) == _lib.E_INVALID
    assert "dspark_plan_pack" in _lib.last_error()


def test_plan_pack_ex_argument_errors():
    tiers = (ctypes.c_int32 * 2)(8, 20)
    base = dict(B=4, gamma=4, kind=0, conf=FAKE, temp=FAKE, mn=1, mx=5, eps=1e-3, lo=0, hi=-1,
                bias=0.5, alpha=FAKE, alen=5, theta=FAKE, tlen=21, lens=FAKE, meta=FAKE, val=FAKE,
                surv=NULL, sweep=NULL, anchors=FAKE, drafts=FAKE,
                tiers=ctypes.cast(tiers, ctypes.c_void_p), ntiers=2, prefix=NULL, cu=FAKE,
                ids=FAKE, req=NULL, pos=NULL, pmeta=FAKE, opt=NULL, stream=NULL)

    def run(opt=None, **kw):
        d = dict(base)
        d.update(kw)
        if opt is not None:
            d["opt"] = ctypes.cast(ctypes.pointer(opt), ctypes.c_void_p)
        return _lib.lib().dspark_plan_pack_ex(*d.values())

    sps1d = dict(cost_mode=_lib.COST_SPS1D, sps_m=FAKE.value, sps=FAKE.value, sps_len=4,
                 align_to_tier=1)
    assert run(gamma=0) == _lib.E_INVALID  # the plan rules still apply
    assert run(ntiers=1) == _lib.E_INVALID  # and the pack rules
    assert run(_lib.PlanOptions(cost_mode=7)) == _lib.E_INVALID
    assert run(_lib.PlanOptions(**{**sps1d, "sps_len": 0})) == _lib.E_INVALID
    assert run(_lib.PlanOptions(**{**sps1d, "sps_len": _lib.MAX_SPS_PROBES + 1})) == _lib.E_INVALID
    assert run(_lib.PlanOptions(**{**sps1d, "sps": None})) == _lib.E_INVALID
    # the additive tables are not needed in 1D mode, but the other rules hold
    assert run(_lib.PlanOptions(**sps1d), alpha=NULL, theta=NULL, alen=0, tlen=0,
               anchors=NULL) == _lib.E_INVALID
    assert "dspark_plan_pack_ex: an input pointer" in _lib.last_error()
    # additive mode still needs its tables
    assert run(_lib.PlanOptions(align_to_tier=1), alpha=NULL) == _lib.E_INVALID


def _pack(tiers, **kw):
    arr = (ctypes.c_int32 * len(tiers))(*tiers)
    a = dict(B=3, gamma=3, lens=FAKE, anchors=FAKE, drafts=FAKE,
             tiers=ctypes.cast(arr, ctypes.c_void_p), ntiers=len(tiers), prefix=NULL, cu=FAKE,
             ids=FAKE, req=NULL, pos=NULL, meta=FAKE, stream=NULL)
    a.update(kw)
    return _lib.lib().dspark_pack(*a.values())


def test_pack_argument_errors():
    assert _pack([4, 8, 12], B=-1) == _lib.E_INVALID
    assert _pack([4, 8, 8]) == _lib.E_INVALID  # not strictly ascending
    assert _pack([4, 8, 11]) == _lib.E_INVALID  # last tier < B * (gamma + 1)
    assert _pack([0, 12]) == _lib.E_INVALID
    assert _pack([12], ntiers=0) == _lib.E_INVALID
    assert _pack(list(range(1, 34))) == _lib.E_INVALID  # more than 32 tiers
    assert _pack([12], ids=NULL) == _lib.E_INVALID
    assert _pack([12], lens=NULL) == _lib.E_INVALID
    assert _pack([12], B=8193, gamma=1) == _lib.E_UNSUPPORTED


def _accept(**kw):
    a = dict(B=2, gamma=4, V=1024, dt=_lib.BF16, logits=FAKE, ld=1024, max_rows=10, cu=FAKE,
             drafts=FAKE, prefix=FAKE, am=FAKE, nc=FAKE, bonus=FAKE, commit=FAKE, out=FAKE,
             newseq=FAKE, mask=NULL, meta=FAKE, ws=ctypes.c_void_p(0x10000), wsb=1 << 20,
             stream=NULL)
    a.update(kw)
    return _lib.lib().dspark_accept(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(V=0), _lib.E_INVALID),
    (dict(V=262145, ld=262152), _lib.E_UNSUPPORTED),
    (dict(dt=5), _lib.E_UNSUPPORTED),
    (dict(ld=1000), _lib.E_INVALID),  # ld < V
    (dict(V=1001, ld=1001), _lib.E_INVALID),  # 2002-byte rows: not a multiple of 16
    (dict(logits=ctypes.c_void_p(0x1008)), _lib.E_INVALID),  # misaligned
    (dict(cu=NULL), _lib.E_INVALID),
    (dict(out=NULL), _lib.E_INVALID),
    (dict(prefix=NULL), _lib.E_INVALID),  # new_seq_lens needs prefix_lens
    (dict(ws=NULL), _lib.E_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x10010)), _lib.E_WORKSPACE),  # not 256-byte aligned
    (dict(wsb=64), _lib.E_WORKSPACE),
    (dict(gamma=65), _lib.E_INVALID),
    (dict(max_rows=-1), _lib.E_INVALID),
])
def test_accept_argument_errors(kw, code):
    assert _accept(**kw) == code


def test_accept_workspace_size():
    f = _lib.lib().dspark_accept_workspace_size
    # 129280 bf16 = 16160 16-byte vectors -> 8 units per row
    assert f(2304, 129280, _lib.BF16) == 2304 * 8 * 8
    assert f(10, 0, _lib.BF16) == 0 and f(-1, 10, _lib.F32) == 0
    assert f(1, 1, _lib.F32) == 256


def test_tv_argument_errors():
    call = _lib.lib().dspark_tv_accept
    ok = dict(B=2, gamma=3, V=1024, dt=_lib.BF16, q=FAKE, ldq=1024, p=FAKE, ldp=1024, rpr=4,
              a=FAKE, s=FAKE, stream=NULL)

    def run(**kw):
        d = dict(ok)
        d.update(kw)
        return call(*d.values())

    assert run(rpr=2) == _lib.E_INVALID
    assert run(ldq=1000) == _lib.E_INVALID
    assert run(q=ctypes.c_void_p(0x1004)) == _lib.E_INVALID
    assert run(a=NULL) == _lib.E_INVALID
    assert run(V=300000, ldq=300000, ldp=300000) == _lib.E_UNSUPPORTED


def test_cap_accept_argument_errors():
    call = _lib.lib().dspark_cap_accept
    ok = dict(B=2, gamma=3, V=1024, dt=_lib.BF16, x=FAKE, ld=1024, lens=FAKE, drafts=FAKE,
              prefix=NULL, am=FAKE, ceil=FAKE, nc=FAKE, bonus=FAKE, commit=FAKE, out=FAKE,
              new_seq=NULL, mask=NULL, meta=FAKE, ws=ctypes.c_void_p(0x100000), wsb=1 << 20,
              stream=NULL)

    def run(**kw):
        d = dict(ok)
        d.update(kw)
        return call(*d.values())

    assert run(gamma=0) == _lib.E_INVALID
    assert run(ld=1000) == _lib.E_INVALID
    assert run(lens=NULL) == _lib.E_INVALID
    assert run(ceil=NULL) == _lib.E_INVALID
    assert run(new_seq=FAKE) == _lib.E_INVALID  # needs prefix_lens
    assert run(dt=7) == _lib.E_UNSUPPORTED
    assert run(wsb=8 * 8 * 4 - 1) == _lib.E_WORKSPACE  # 8 rows, 1 unit each -> 256 bytes
    assert run(ws=ctypes.c_void_p(0x100010)) == _lib.E_WORKSPACE


def test_scatter_argument_errors():
    call = _lib.lib().dspark_scatter_to_strided
    ok = dict(B=2, stride=4, cu=FAKE, max_rows=8, src=FAKE, src_ld=4096, dst=FAKE, dst_ld=4096,
              row_bytes=4000, meta=FAKE, stream=NULL)

    def run(**kw):
        d = dict(ok)
        d.update(kw)
        return call(*d.values())

    assert run(stride=0) == _lib.E_INVALID
    assert run(stride=_lib.MAX_GAMMA + 2) == _lib.E_INVALID
    assert run(row_bytes=0) == _lib.E_INVALID
    assert run(row_bytes=4097) == _lib.E_INVALID  # above a row stride
    assert run(src_ld=4104) == _lib.E_INVALID  # not a multiple of 16
    assert run(dst=ctypes.c_void_p(0x1008)) == _lib.E_INVALID
    assert run(cu=NULL) == _lib.E_INVALID
    assert run(max_rows=-1) == _lib.E_INVALID


def test_sts_fit_argument_errors():
    call = _lib.lib().dspark_sts_fit
    grid = (ctypes.c_float * 3)(0.5, 1.0, 2.0)
    bad_grid = (ctypes.c_float * 3)(0.5, 0.0, 2.0)
    ok = dict(N=100, gamma=4, z=FAKE, mask=FAKE, grid=ctypes.cast(grid, ctypes.c_void_p), nt=3,
              nb=15, temps=FAKE, idx=FAKE, ece=FAKE, brier=FAKE, eg=NULL, surv=NULL,
              ws=ctypes.c_void_p(0x100000), wsb=0, stream=NULL)

    def run(**kw):
        d = dict(ok)
        d.update(kw)
        return call(*d.values())

    assert run(N=-1) == _lib.E_INVALID
    assert run(N=_lib.STS_MAX_RECORDS + 1) == _lib.E_UNSUPPORTED
    assert run(gamma=0) == _lib.E_INVALID
    assert run(nt=0) == _lib.E_INVALID
    assert run(nt=_lib.STS_MAX_GRID + 1) == _lib.E_INVALID
    assert run(grid=ctypes.cast(bad_grid, ctypes.c_void_p)) == _lib.E_INVALID
    assert run(nb=0) == _lib.E_INVALID and run(nb=_lib.STS_MAX_BINS + 1) == _lib.E_INVALID
    assert run(z=NULL) == _lib.E_INVALID
    assert run(temps=NULL) == _lib.E_INVALID
    assert run() == _lib.E_WORKSPACE  # 0 bytes given
    size = _lib.lib().dspark_sts_workspace_size
    # two survival buffers of 100 floats, then three summed-histogram buffers
    # of 3 x 31 int64 words (one region), each region 256-byte aligned
    assert size(100, 4, 3, 15) == 2 * 512 + 2304
    # 300 records: only the survival buffers grow
    assert size(300, 4, 3, 15) == 2 * 1280 + 2304
    # 4194304 records, one candidate, one bin: three buffers of 3 words
    assert size(4194304, 1, 1, 1) == 2 * 4 * 4194304 + 256
    assert size(0, 4, 3, 15) > 0 and size(-1, 4, 3, 15) == 0 and size(10, 4, 129, 15) == 0


# ---------------------------------------------------------------- sigmoid logic on the CPU

def _host_sigmoid(x, force_slow=False):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    slow = np.zeros(x.shape, dtype=np.uint8)
    _lib.hostcheck().dspark_hostcheck_sigmoid(x.ctypes.data, y.ctypes.data, slow.ctypes.data,
                                              x.size, 1 if force_slow else 0)
    return y, slow


def test_device_sigmoid_fast_path_matches_oracle():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.normal(0, 4, 200000), rng.uniform(-104, 18, 50000),
        [0.0, -0.0, 17.3, 17.33, 17.34, 17.5, -87.3, -90.0, -103.9, -104.0, np.inf, -np.inf],
    ]).astype(np.float32)
    y, _ = _host_sigmoid(x)
    assert np.array_equal(y.view(np.uint32), sigmoid32(x).view(np.uint32))


def test_device_sigmoid_exact_path_matches_oracle():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.normal(0, 5, 3000), rng.uniform(-103.9, 17.4, 1000)]).astype(np.float32)
    y, slow = _host_sigmoid(x, force_slow=True)
    assert slow[(x > -104) & (x < 17.5)].all()
    assert np.array_equal(y.view(np.uint32), sigmoid32(x).view(np.uint32))


def test_inputs_that_reach_the_exact_path():
    # scan random inputs until the fast path declines some; those must still be exact
    rng = np.random.default_rng(7)
    hits = []
    for _ in range(40):
        x = rng.uniform(-30, 18, 1_000_000).astype(np.float32)
        y, slow = _host_sigmoid(x)
        idx = np.flatnonzero(slow)
        hits.extend((x[i], y[i]) for i in idx)
        if len(hits) >= 8:
            break
    assert len(hits) >= 1
    for xv, yv in hits:
        assert np.float32(yv).view(np.uint32) == nearest_f32(sigmoid_decimal(float(xv))).view(np.uint32)


def test_accept_sampling_argument_errors():
    call = _lib.lib().dspark_accept_sampling
    ok = dict(B=4, gamma=3, V=1000, dt=_lib.BF16, tgt=FAKE, ld=1000, max_rows=16, cu=FAKE,
              drf=FAKE, ld_q=1000, drafts=FAKE, temps=FAKE, ra=FAKE, rs=FAKE, prefix=NULL,
              nc=FAKE, bonus=FAKE, commit=FAKE, out=FAKE, new_seq=NULL, meta=FAKE,
              ws=ctypes.c_void_p(0x100000), wsb=0, stream=NULL)

    def run(**kw):
        d = dict(ok)
        d.update(kw)
        return call(*d.values())

    assert run(B=-1) == _lib.E_INVALID
    assert run(gamma=0) == _lib.E_INVALID and run(gamma=65) == _lib.E_INVALID
    assert run(dt=7) == _lib.E_UNSUPPORTED
    assert run(V=0) == _lib.E_INVALID and run(V=_lib.MAX_VOCAB + 1) == _lib.E_UNSUPPORTED
    assert run(ld=999) == _lib.E_INVALID and run(ld_q=999) == _lib.E_INVALID
    assert run(ld=1001) == _lib.E_INVALID  # 2002 bytes: not a multiple of 16
    assert run(tgt=ctypes.c_void_p(0x1002)) == _lib.E_INVALID
    assert run(drf=NULL) == _lib.E_INVALID
    assert run(temps=NULL) == _lib.E_INVALID and run(rs=NULL) == _lib.E_INVALID
    assert run(new_seq=FAKE) == _lib.E_INVALID  # needs prefix_lens
    assert run(max_rows=2**31 - 8) == _lib.E_UNSUPPORTED  # + B * gamma overflows
    assert run() == _lib.E_WORKSPACE
    size = _lib.lib().dspark_accept_sampling_workspace_size
    # 9 + 12 slots, one chunk of 125 vectors: 21 keys and 21 sums, 4 requests
    # of 2 x 2 residual sums, 4 jobs of 48 bytes
    assert size(4, 3, 1000, _lib.BF16) == 256 + 256 + 256 + 256
    # V = 129280 bf16: 16160 vectors in 8 chunks; 4 * 17 slots; residual sums
    # per (request, chunk, half chunk)
    assert size(4, 8, 129280, _lib.BF16) == 2 * (4 * 17 * 8 * 8) + 1024 + 256  # 4352 = 17 * 256
    assert size(0, 3, 100, _lib.F32) == 256  # one job slot, no partials
    assert size(-1, 3, 100, _lib.F32) == 0 and size(4, 65, 100, _lib.F32) == 0
    assert size(4, 3, 0, _lib.F32) == 0 and size(4, 3, 100, 7) == 0


def test_accept_noalloc_argument_errors():
    call = _lib.lib().dspark_accept_noalloc
    ok = dict(B=2, gamma=4, V=1024, dt=_lib.BF16, logits=FAKE, ld=1024, max_rows=10, cu=FAKE,
              drafts=FAKE, prefix=FAKE, am=FAKE, nc=FAKE, bonus=FAKE, commit=FAKE, out=FAKE,
              newseq=FAKE, mask=NULL, meta=FAKE, stream=NULL)

    def run(**kw):
        d = dict(ok)
        d.update(kw)
        return call(*d.values())

    assert run(V=0) == _lib.E_INVALID
    assert run(cu=NULL) == _lib.E_INVALID
    assert run(logits=ctypes.c_void_p(0x1008)) == _lib.E_INVALID
    # partials beyond the 1 MiB array are refused before any launch: at V =
    # 129280 bf16 (8 units per row) that is max_rows > 16384; at V = 262144
    # float32 (32 units) max_rows > 4096
    assert run(V=129280, ld=129280, max_rows=16385) == _lib.E_WORKSPACE
    assert run(V=262144, ld=262144, dt=_lib.F32, max_rows=4097) == _lib.E_WORKSPACE
    assert b"1048576" in _lib.lib().dspark_last_error()
    f = _lib.lib().dspark_accept_workspace_size
    assert f(16384, 129280, _lib.BF16) == 1 << 20 and f(4096, 262144, _lib.F32) == 1 << 20


def test_m0_check_of_the_build():
    from dspark_verify_scheduling_amd.build import check_m0_use

    good = "\t;;#ASMSTART\n\ts_mov_b32 m0, s14\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v1, s[42:43]\n\t;;#ASMEND\n"
    check_m0_use(good)
    for bad in ("\ts_mov_b32 m0, -1\n\tds_read_b32 v0, v1\n",
                good + "\ts_mov_b32 m0, s3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v1, s[4:5]\n",
                "\t;;#ASMSTART\n\ts_mov_b32 m0, s14\n\ts_add_u32 s1, s1, 1\n\tglobal_load_lds_dwordx4 v1, s[2:3]\n\t;;#ASMEND\n",
                "\tv_readlane_b32 s0, v1, m0\n"):
        with pytest.raises(RuntimeError):
            check_m0_use(bad)
