"""dspark_accept_noalloc (the accept without a workspace, for callers that
cannot allocate) against dspark_accept, through the C ABI: bit for bit on
every output, on two calls in a row, the second with a smaller input (fewer
requests and rows, another vocabulary and element type), so the second reads
the library's scratch array after the first left its partials there."""

import numpy as np
import pytest
import torch

import dspark_verify_scheduling_amd as dv
import oracle
from workloads import make
from _gpu import DEV, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(hip):
    return hip


def _layout(cfg):
    w = make(cfg)
    p = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len, w.max_len,
                    w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
    lens = p["verify_lens"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    max_rows = int(w.tiers[np.searchsorted(w.tiers, total)])
    rows = np.concatenate([w.target[r, :lens[r]] for r in range(w.B)])
    dt = dv.BF16 if w.dtype == "bf16" else dv.F32
    buf = np.zeros((max_rows, w.V), rows.dtype)
    buf[:total] = rows
    if dt == dv.BF16:
        logits = torch.from_numpy(buf.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        logits = torch.from_numpy(buf).to(DEV)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return dict(B=w.B, gamma=w.gamma, V=w.V, dt=dt, logits=logits, max_rows=max_rows,
                cu=t(cu), drafts=t(w.drafts), prefix=t(w.prefix_lens), total=total)


def _call(fn, c):
    out = dv.alloc_accept_outputs(c["B"], c["gamma"], c["max_rows"], c["V"], c["dt"], DEV)
    for x in out[:-1]:
        if x is not None:
            x.fill_(-7 if x.dtype == torch.int32 else 0x5A)
    fn(c["B"], c["gamma"], c["V"], c["dt"], c["logits"], c["V"], c["max_rows"], c["cu"],
       c["drafts"], c["prefix"], out)
    torch.cuda.synchronize()
    return out


def _same(a, b, total):
    assert torch.equal(a.row_argmax[:total], b.row_argmax[:total])
    for name in ("num_correct", "bonus", "commit_lens", "out_tokens", "new_seq_lens",
                 "prefix_mask", "accept_meta"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def test_noalloc_equals_accept_on_two_calls_in_a_row():
    big = _layout(3)  # B = 256, gamma = 8, V = 129280 bf16, 755 rows in a 1024-row tier
    say(f"noalloc call 1: B={big['B']} V={big['V']} rows={big['total']} max_rows={big['max_rows']}")
    got = _call(dv.dspark_accept_noalloc, big)
    ref = _call(dv.dspark_accept, big)
    _same(got, ref, big["total"])
    assert got.accept_meta.tolist() == [big["total"], 0]
    small = _layout(1)  # B = 8, V = 32000 float32
    say(f"noalloc call 2: B={small['B']} V={small['V']} rows={small['total']}")
    got2 = _call(dv.dspark_accept_noalloc, small)
    ref2 = _call(dv.dspark_accept, small)
    _same(got2, ref2, small["total"])
    assert got2.accept_meta.tolist() == [small["total"], 0]
    # and the first input again, after the smaller call
    got3 = _call(dv.dspark_accept_noalloc, big)
    _same(got3, ref, big["total"])
