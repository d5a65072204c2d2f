"""GPU parity for the strided-layout entry points: cap-accept and the scatter
of packed rows back to stride, through the C ABI, against the CPU oracle.

Bar: every output is bit-exact (row argmax, ceiling, num_correct, bonus,
commit, out_tokens, new_seq, prefix_mask, meta; scattered bytes; untouched
destination rows keep their sentinel).
"""

import numpy as np
import pytest
import torch

import dspark_verify_scheduling_amd as dv
import oracle
from oracle.accept import as_f32_rows
from workloads import make
from _gpu import DEV, accept, gather_packed, logits_up, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(hip):
    return hip


_WL = {}


def _workload(cfg):
    if cfg not in _WL:
        say(f"generating workload cfg{cfg}")
        _WL.clear()
        _WL[cfg] = make(cfg)
    return _WL[cfg]


def _eq(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    bad = a != b
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} mismatches, first at {idx.tolist()}: "
                             f"gpu={a[tuple(idx[0])]} oracle={b[tuple(idx[0])]}")


def cap_accept(B, gamma, V, dt, rows, ld, lens, drafts, prefix=None, tag=""):
    say(f"cap_accept {tag} B={B} gamma={gamma} V={V} ld={ld} dt={dt}")
    x = logits_up(rows, dt) if B else logits_up(np.zeros((1, ld), np.float32), 0)
    outs = dv.alloc_cap_accept_outputs(B, gamma, V, dt, DEV, new_seq=prefix is not None)
    outs.row_argmax.fill_(-7)
    dv.dspark_cap_accept(B, gamma, V, dt, x, ld, up(np.asarray(lens, np.int32)),
                         up(np.asarray(drafts, np.int32).reshape(B, gamma)),
                         up(np.asarray(prefix, np.int32)) if prefix is not None else None, outs)
    torch.cuda.synchronize()
    return {
        "row_argmax": outs.row_argmax.cpu().numpy()[: B * (gamma + 1)],
        "ceiling": outs.ceiling.cpu().numpy(),
        "num_correct": outs.num_correct.cpu().numpy(),
        "bonus": outs.bonus.cpu().numpy(),
        "commit": outs.commit_lens.cpu().numpy(),
        "out_tokens": outs.out_tokens.cpu().numpy(),
        "new_seq": outs.new_seq_lens.cpu().numpy() if outs.new_seq_lens is not None else None,
        "prefix_mask": outs.prefix_mask.cpu().numpy(),
        "meta": outs.accept_meta.cpu().numpy(),
    }


def _check_cap(got, ref):
    for k in ("row_argmax", "ceiling", "num_correct", "bonus", "commit", "out_tokens",
              "prefix_mask", "meta"):
        _eq(got[k], ref[k], k)
    if got["new_seq"] is not None:
        _eq(got["new_seq"], ref["new_seq"], "new_seq")


def _strided_rows(w):
    return w.target.reshape(w.B * (w.gamma + 1), w.V)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_cap_accept_parity_planned(cfg):
    w = _workload(cfg)
    lens = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                       w.max_len, w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)["verify_lens"]
    dt = dv.BF16 if w.dtype == "bf16" else dv.F32
    rows = _strided_rows(w)
    got = cap_accept(w.B, w.gamma, w.V, dt, rows, w.V, lens, w.drafts, w.prefix_lens,
                     tag=f"cfg{cfg} planned")
    ref = oracle.cap_accept(w.B, w.gamma, rows, w.dtype, lens, w.drafts, w.prefix_lens)
    _check_cap(got, ref)
    say(f"cfg{cfg}: committed {int(ref['num_correct'].sum())} drafts of a ceiling of "
        f"{int(ref['ceiling'].sum())}")


def test_cap_accept_commits_what_compact_commits():
    """Cap-accept on the strided rows and compact accept on the packed rows
    (both on the GPU) commit the same tokens."""
    w = _workload(2)
    rng = np.random.default_rng(77)
    lens = rng.integers(1, w.gamma + 2, w.B).astype(np.int32)
    dt = dv.BF16
    got_cap = cap_accept(w.B, w.gamma, w.V, dt, _strided_rows(w), w.V, lens, w.drafts,
                         w.prefix_lens, tag="cfg2 random lens")
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rows = gather_packed(w.target, cu, lens, int(cu[-1]))
    got_cmp = accept(w.B, w.gamma, w.V, dt, rows, w.V, cu, w.drafts, w.prefix_lens,
                     tag="cfg2 compact")
    for k in ("num_correct", "bonus", "commit", "out_tokens", "prefix_mask", "new_seq"):
        _eq(got_cap[k], got_cmp[k], k)
    assert np.all(got_cap["ceiling"] >= got_cap["num_correct"])


@pytest.mark.parametrize("V,ld,dt", [(1001, 1008, dv.BF16), (7, 8, dv.F32), (32000, 32004, dv.F32)])
def test_cap_accept_bad_lengths_and_shapes(V, ld, dt):
    rng = np.random.default_rng(V)
    B, gamma = 37, 5
    x = rng.normal(0, 2, (B * (gamma + 1), ld)).astype(np.float32)
    x[5, :V] = 0.0  # a constant row: index 0
    rows = x if dt == dv.F32 else (x.view(np.uint32) >> 16).astype(np.uint16)
    am = oracle.row_argmax(as_f32_rows(rows[:, :V], "bf16" if dt else "f32"))
    drafts = np.where(rng.random((B, gamma)) < 0.7, am.reshape(B, gamma + 1)[:, :gamma],
                      rng.integers(0, V, (B, gamma))).astype(np.int32)
    lens = rng.integers(0, gamma + 3, B).astype(np.int32)  # 0 and gamma + 2 are invalid
    prefix = rng.integers(0, 1000, B).astype(np.int32)
    got = cap_accept(B, gamma, V, dt, rows, ld, lens, drafts, prefix, tag=f"V={V} ld={ld}")
    ref = oracle.cap_accept(B, gamma, rows[:, :V], "bf16" if dt else "f32", lens, drafts, prefix)
    assert ref["meta"][1] == oracle.DATA_BAD_LENS
    _check_cap(got, ref)


def test_cap_accept_gamma_64():
    """gamma = 64: 65 strided rows per request, a ceiling of up to 64."""
    rng = np.random.default_rng(640)
    B, gamma, V = 4, 64, 1500
    x = rng.normal(0, 2, (B * (gamma + 1), V)).astype(np.float32)
    am = oracle.row_argmax(x).reshape(B, gamma + 1)
    drafts = am[:, :gamma].copy()
    drafts[1, 40] = (drafts[1, 40] + 1) % V  # request 1 misses at draft 41
    drafts[3, 0] = (drafts[3, 0] + 1) % V  # request 3 misses at once
    lens = np.array([65, 65, 12, 65], np.int32)
    prefix = rng.integers(0, 1000, B).astype(np.int32)
    got = cap_accept(B, gamma, V, dv.F32, x, V, lens, drafts, prefix, tag="gamma=64")
    ref = oracle.cap_accept(B, gamma, x, "f32", lens, drafts, prefix)
    assert ref["ceiling"].tolist() == [64, 40, 64, 0]
    assert ref["num_correct"].tolist() == [64, 40, 11, 0]
    _check_cap(got, ref)


def test_cap_accept_empty_batch():
    got = cap_accept(0, 3, 64, dv.F32, None, 64, np.zeros(0, np.int32),
                     np.zeros((0, 3), np.int32), tag="B=0")
    assert got["meta"].tolist() == [0, 0]


# ---------------------------------------------------------------- scatter

def scatter(B, stride, cu, packed_np, row_elems, dst_init_np, tag=""):
    say(f"scatter {tag} B={B} stride={stride} rows={packed_np.shape[0]} row_elems={row_elems}")
    src = torch.from_numpy(np.ascontiguousarray(packed_np)).to(DEV)
    dst = torch.from_numpy(np.ascontiguousarray(dst_init_np)).to(DEV)
    meta = torch.empty(2, dtype=torch.int32, device=DEV)
    dv.dspark_scatter_to_strided(B, stride, up(np.asarray(cu, np.int32)), src, dst, row_elems, meta)
    torch.cuda.synchronize()
    return dst.cpu().numpy(), meta.cpu().numpy()


def _scatter_case(rng, B, stride, width, ld_src, ld_dst, dtype, lens=None, pad=3):
    if lens is None:
        lens = rng.integers(1, stride + 1, B)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(cu[-1]) + pad
    packed = rng.integers(-2**15, 2**15, (n, ld_src)).astype(dtype)
    init = np.full((B * stride, ld_dst), -3, dtype=dtype)
    return cu, packed, init


@pytest.mark.parametrize("width,ld_src,ld_dst,dtype", [
    (129280, 129280, 129280, np.int16),   # bf16 logits, V = 129280
    (7168, 7168, 7176, np.int16),         # bf16 hidden states, H = 7168, padded destination
    (1001, 1008, 1016, np.int16),         # 2002 bytes: a 2-byte tail
    (3, 8, 8, np.int16),                  # 6 bytes: tail only
    (32000, 32000, 32004, np.float32),    # fp32 logits
])
def test_scatter_parity(width, ld_src, ld_dst, dtype):
    rng = np.random.default_rng(width)
    B, stride = 29, 9
    cu, packed, init = _scatter_case(rng, B, stride, width, ld_src, ld_dst, dtype)
    got, meta = scatter(B, stride, cu, packed, width, init, tag=f"width={width}")
    ref, ref_meta = oracle.scatter_to_strided(B, stride, cu, packed[:, :width], init[:, :width],
                                              max_rows=packed.shape[0])
    _eq(meta, ref_meta, "meta")
    _eq(got[:, :width], ref, "strided rows")
    assert np.all(got[:, width:] == -3), "bytes past row_bytes were written"


def test_scatter_long_requests():
    """stride 65 (gamma = 64): requests of 1..65 rows, lengths on both sides of
    the eight-row batches, and a row width with a byte tail."""
    rng = np.random.default_rng(65)
    B, stride, width = 9, 65, 1025
    lens = np.array([65, 64, 17, 16, 9, 8, 7, 1, 33], np.int64)
    cu, packed, init = _scatter_case(rng, B, stride, width, 1032, 1040, np.int16, lens=lens)
    got, meta = scatter(B, stride, cu, packed, width, init, tag="stride=65")
    ref, ref_meta = oracle.scatter_to_strided(B, stride, cu, packed[:, :width], init[:, :width],
                                              max_rows=packed.shape[0])
    assert meta.tolist() == ref_meta.tolist() == [int(cu[-1]), 0]
    _eq(got[:, :width], ref, "strided rows")
    _eq(got[:, width:], init[:, width:], "destination padding")


def test_scatter_planned_layout_round_trip():
    """The planned cfg3 layout: scatter the packed target rows back and find
    the original strided rows at every verified slot."""
    w = _workload(3)
    lens = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                       w.max_len, w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)["verify_lens"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tier = int(oracle.pack(w.B, w.gamma, lens, w.anchors, w.drafts, w.tiers)["meta"][1])
    packed = gather_packed(w.target, cu, lens, tier).view(np.int16)
    stride = w.gamma + 1
    init = np.full((w.B * stride, w.V), 0x7FC1, dtype=np.int16)
    got, meta = scatter(w.B, stride, cu, packed, w.V, init, tag="cfg3 planned")
    assert meta.tolist() == [int(cu[-1]), 0]
    strided = w.target.reshape(w.B * stride, w.V).view(np.int16)
    for r in range(w.B):
        base = r * stride
        assert np.array_equal(got[base: base + lens[r]], strided[base: base + lens[r]])
        assert np.all(got[base + lens[r]: base + stride] == 0x7FC1)


def test_scatter_malformed_and_empty():
    rng = np.random.default_rng(5)
    packed = rng.integers(-100, 100, (6, 32)).astype(np.int16)
    init = np.full((8, 32), -1, dtype=np.int16)
    cu = np.array([0, 2, 2, 5, 7], np.int32)  # empty, too long, past max_rows
    got, meta = scatter(4, 2, cu, packed, 32, init, tag="malformed")
    ref, ref_meta = oracle.scatter_to_strided(4, 2, cu, packed, init, max_rows=6)
    _eq(meta, ref_meta, "meta")
    _eq(got, ref, "strided rows")
    got, meta = scatter(0, 4, np.zeros(1, np.int32), packed, 32, init, tag="B=0")
    assert meta.tolist() == [0, 0]
    assert np.all(got == -1)
