"""Helpers for the GPU tests: upload host inputs, call one entry point through
the binding (and so through the C ABI), synchronize, return numpy outputs.

Every step prints the case it is about to run, so a run that dies on the GPU
still names its last case.
"""

from __future__ import annotations

import numpy as np
import torch

import dspark_verify_scheduling_amd as dv

DEV = "cuda"


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def up(a, dtype=None):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def logits_up(rows: np.ndarray, dt: int) -> torch.Tensor:
    """Upload logit rows given as float32 or bf16 bit patterns (uint16)."""
    rows = np.ascontiguousarray(rows)
    if dt == dv.BF16:
        return torch.from_numpy(rows.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(rows.astype(np.float32, copy=False)).to(DEV)


def plan(B, gamma, kind, conf, temps, min_len, max_len, eps, b_lo, b_hi, bias, alpha, theta,
         sweep=True, tag=""):
    say(f"plan {tag} B={B} gamma={gamma} kind={kind}")
    out = dv.alloc_plan_outputs(B, gamma, DEV, survival=True, sweep=sweep)
    conf_t = up(np.asarray(conf, np.float32).reshape(B, gamma))
    temps_t = up(np.asarray(temps, np.float32)) if temps is not None else None
    dv.dspark_plan(B, gamma, kind, conf_t, temps_t, min_len, max_len, float(eps), b_lo, b_hi,
                   float(bias), up(np.asarray(alpha, np.float32)), up(np.asarray(theta, np.float32)),
                   out)
    torch.cuda.synchronize()
    return {
        "verify_lens": out.verify_lens.cpu().numpy(),
        "meta": out.plan_meta.cpu().numpy(),
        "val": out.plan_val.cpu().numpy(),
        "survival": out.survival_out.cpu().numpy(),
        "sweep": out.sweep_out.cpu().numpy() if sweep else None,
    }


def pack(B, gamma, lens, anchors, drafts, tiers, prefix=None, req=True, pos=True, tag=""):
    say(f"pack {tag} B={B} gamma={gamma}")
    cap = int(tiers[-1])
    out = dv.alloc_pack_outputs(B, cap, DEV, req=req, pos=pos)
    for t in (out.packed_ids, out.packed_req, out.packed_pos):
        if t is not None:
            t.fill_(-7)  # sentinel: rows beyond the tier must stay untouched
    dv.dspark_pack(B, gamma, up(np.asarray(lens, np.int32)), up(np.asarray(anchors, np.int32)),
                   up(np.asarray(drafts, np.int32).reshape(B, gamma)), tiers,
                   up(np.asarray(prefix, np.int32)) if prefix is not None else None, out)
    torch.cuda.synchronize()
    return {
        "cu_seqlens": out.cu_seqlens.cpu().numpy(),
        "ids": out.packed_ids.cpu().numpy(),
        "req": out.packed_req.cpu().numpy() if req else None,
        "pos": out.packed_pos.cpu().numpy() if pos else None,
        "meta": out.pack_meta.cpu().numpy(),
    }


def plan_pack(B, gamma, kind, conf, temps, min_len, max_len, eps, b_lo, b_hi, bias, alpha,
              theta, anchors, drafts, tiers, prefix=None, tag=""):
    say(f"plan_pack {tag} B={B} gamma={gamma} kind={kind}")
    cap = int(tiers[-1])
    po = dv.alloc_plan_outputs(B, gamma, DEV, survival=True, sweep=True)
    ko = dv.alloc_pack_outputs(B, cap, DEV)
    for t in (ko.packed_ids, ko.packed_req, ko.packed_pos):
        t.fill_(-7)
    temps_t = up(np.asarray(temps, np.float32)) if temps is not None else None
    dv.dspark_plan_pack(B, gamma, kind, up(np.asarray(conf, np.float32).reshape(B, gamma)), temps_t,
                        min_len, max_len, float(eps), b_lo, b_hi, float(bias),
                        up(np.asarray(alpha, np.float32)), up(np.asarray(theta, np.float32)), po,
                        up(np.asarray(anchors, np.int32)),
                        up(np.asarray(drafts, np.int32).reshape(B, gamma)), tiers,
                        up(np.asarray(prefix, np.int32)) if prefix is not None else None, ko)
    torch.cuda.synchronize()
    return ({"verify_lens": po.verify_lens.cpu().numpy(), "meta": po.plan_meta.cpu().numpy(),
             "val": po.plan_val.cpu().numpy(), "survival": po.survival_out.cpu().numpy(),
             "sweep": po.sweep_out.cpu().numpy()},
            {"cu_seqlens": ko.cu_seqlens.cpu().numpy(), "ids": ko.packed_ids.cpu().numpy(),
             "req": ko.packed_req.cpu().numpy(), "pos": ko.packed_pos.cpu().numpy(),
             "meta": ko.pack_meta.cpu().numpy()})


def plan_pack_ex(B, gamma, kind, conf, temps, min_len, max_len, eps, b_lo, b_hi, bias, alpha,
                 theta, anchors, drafts, tiers, prefix=None, cost_mode=0, sps_m=None, sps=None,
                 align=False, tag=""):
    say(f"plan_pack_ex {tag} B={B} gamma={gamma} kind={kind} cost_mode={cost_mode} align={align}")
    cap = int(tiers[-1])
    po = dv.alloc_plan_outputs(B, gamma, DEV, survival=True, sweep=True)
    ko = dv.alloc_pack_outputs(B, cap, DEV)
    for t in (ko.packed_ids, ko.packed_req, ko.packed_pos):
        t.fill_(-7)
    temps_t = up(np.asarray(temps, np.float32)) if temps is not None else None
    dv.dspark_plan_pack_ex(
        B, gamma, kind, up(np.asarray(conf, np.float32).reshape(B, gamma)), temps_t, min_len,
        max_len, float(eps), b_lo, b_hi, float(bias),
        up(np.asarray(alpha, np.float32)) if alpha is not None else None,
        up(np.asarray(theta, np.float32)) if theta is not None else None, po,
        up(np.asarray(anchors, np.int32)), up(np.asarray(drafts, np.int32).reshape(B, gamma)),
        tiers, up(np.asarray(prefix, np.int32)) if prefix is not None else None, ko,
        cost_mode=cost_mode, sps_m=up(np.asarray(sps_m, np.int32)) if sps_m is not None else None,
        sps=up(np.asarray(sps, np.float32)) if sps is not None else None, align_to_tier=align)
    torch.cuda.synchronize()
    return ({"verify_lens": po.verify_lens.cpu().numpy(), "meta": po.plan_meta.cpu().numpy(),
             "val": po.plan_val.cpu().numpy(), "survival": po.survival_out.cpu().numpy(),
             "sweep": po.sweep_out.cpu().numpy()},
            {"cu_seqlens": ko.cu_seqlens.cpu().numpy(), "ids": ko.packed_ids.cpu().numpy(),
             "req": ko.packed_req.cpu().numpy(), "pos": ko.packed_pos.cpu().numpy(),
             "meta": ko.pack_meta.cpu().numpy()})


def accept(B, gamma, V, dt, rows, ld, cu, drafts, prefix=None, max_rows=None, outs=None,
           logits_t=None, tag=""):
    """rows: host array [max_rows, ld] (float32 or bf16 bits), or pass logits_t."""
    if max_rows is None:
        max_rows = rows.shape[0]
    say(f"accept {tag} B={B} gamma={gamma} V={V} ld={ld} max_rows={max_rows} dt={dt}")
    if logits_t is None:
        logits_t = logits_up(rows, dt)
    if outs is None:
        outs = dv.alloc_accept_outputs(B, gamma, max_rows, V, dt, DEV,
                                       new_seq=prefix is not None, mask=True)
    outs.row_argmax.fill_(-7)
    dv.dspark_accept(B, gamma, V, dt, logits_t, ld, max_rows, up(np.asarray(cu, np.int32)),
                     up(np.asarray(drafts, np.int32).reshape(B, gamma)),
                     up(np.asarray(prefix, np.int32)) if prefix is not None else None, outs)
    torch.cuda.synchronize()
    return {
        "row_argmax": outs.row_argmax.cpu().numpy(),
        "num_correct": outs.num_correct.cpu().numpy(),
        "bonus": outs.bonus.cpu().numpy(),
        "commit": outs.commit_lens.cpu().numpy(),
        "out_tokens": outs.out_tokens.cpu().numpy(),
        "new_seq": outs.new_seq_lens.cpu().numpy() if outs.new_seq_lens is not None else None,
        "prefix_mask": outs.prefix_mask.cpu().numpy(),
        "meta": outs.accept_meta.cpu().numpy(),
    }


def tv(B, gamma, V, dt, q_t, ld_q, p_t, ld_p, rows_per_req, tag=""):
    say(f"tv {tag} B={B} gamma={gamma} V={V}")
    a = torch.empty(B, gamma, dtype=torch.float32, device=DEV)
    s = torch.empty(B, gamma, dtype=torch.float32, device=DEV)
    dv.dspark_tv_accept(B, gamma, V, dt, q_t, ld_q, p_t, ld_p, rows_per_req, a, s)
    torch.cuda.synchronize()
    return a.cpu().numpy(), s.cpu().numpy()


def gather_packed(strided: np.ndarray, cu: np.ndarray, lens: np.ndarray, capacity: int,
                  pad_value=None) -> np.ndarray:
    """Stand-in for the target forward: packed row cu[r] + j holds strided row [r, j].

    Rows past the total are filled with ``pad_value`` (default: NaN bit
    patterns), so a kernel that read them would be caught."""
    B, _, V = strided.shape
    out = np.empty((capacity, V), dtype=strided.dtype)
    if pad_value is None:
        pad_value = np.uint16(0x7FC1) if strided.dtype == np.uint16 else np.float32(np.nan)
    out[:] = pad_value
    req = np.repeat(np.arange(B), lens)
    j = np.arange(int(cu[-1])) - np.repeat(cu[:-1], lens)
    out[: int(cu[-1])] = strided[req, j]
    return out
