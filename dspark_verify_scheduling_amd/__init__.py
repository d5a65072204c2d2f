"""MI355X (gfx950) DSpark per-step verify path: Python binding of libdspark.

The functions below carry the names of the C entry points in
``include/dspark.h`` and only marshal arguments. They check that each tensor
is a contiguous CUDA tensor of the right dtype and size, pass raw pointers and
the current HIP stream, and raise ``DsparkError`` on a non-OK status. Every
step of the computation runs in the library's HIP kernels. PyTorch supplies
device memory and streams.

``alloc_*`` helpers allocate output tensors for convenience. The library
itself never allocates.
"""

from __future__ import annotations

from typing import NamedTuple, Optional, Sequence

import torch

from . import _lib
from ._lib import (
    BF16, COST_ADDITIVE, COST_SPS1D, DATA_BAD_CONF, DATA_BAD_COST, DATA_BAD_LENS,
    DATA_BAD_LOGITS, F32, IN_COND,
    IN_CONF_LOGITS,
    IN_SURVIVAL, MAX_BATCH, MAX_CANDIDATES, MAX_GAMMA, MAX_TIERS, MAX_VOCAB, DsparkError,
)

__all__ = [
    "load", "dspark_plan", "dspark_pack", "dspark_plan_pack", "dspark_plan_pack_ex",
    "dspark_accept", "dspark_accept_noalloc", "dspark_tv_accept", "COST_ADDITIVE", "COST_SPS1D",
    "dspark_cap_accept", "dspark_scatter_to_strided", "dspark_accept_workspace_size",
    "alloc_plan_outputs", "alloc_pack_outputs", "alloc_accept_outputs",
    "alloc_cap_accept_outputs", "dspark_sts_fit", "dspark_sts_workspace_size", "DsparkError", "F32", "BF16", "IN_CONF_LOGITS", "IN_COND",
    "IN_SURVIVAL", "DATA_BAD_COST", "DATA_BAD_CONF", "DATA_BAD_LENS", "DATA_BAD_LOGITS",
    "dspark_accept_sampling", "dspark_accept_sampling_workspace_size",
    "alloc_sampling_outputs",
]


def load():
    """Load libdspark.so (raises if it is not built)."""
    return _lib.lib()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype, numel: int, required: bool = True):
    if t is None:
        if required and numel > 0:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:  # (cheaper than t.device.type)
        raise ValueError(f"{name} must be a CUDA tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _logit_dtype(dt: int):
    if dt == BF16:
        return torch.bfloat16
    if dt == F32:
        return torch.float32
    raise ValueError(f"unknown dtype code {dt}")


# ------------------------------------------------------------------ plan

class PlanOutputs(NamedTuple):
    verify_lens: torch.Tensor  # [B] int32
    plan_meta: torch.Tensor  # [4] int32
    plan_val: torch.Tensor  # [2] float64
    survival_out: Optional[torch.Tensor]  # [B, gamma] float32
    sweep_out: Optional[torch.Tensor]  # [B*gamma+1, 2] float64


def alloc_plan_outputs(B: int, gamma: int, device, survival=True, sweep=False) -> PlanOutputs:
    return PlanOutputs(
        torch.empty(B, dtype=torch.int32, device=device),
        torch.empty(4, dtype=torch.int32, device=device),
        torch.empty(2, dtype=torch.float64, device=device),
        torch.empty(B, gamma, dtype=torch.float32, device=device) if survival else None,
        torch.empty(B * gamma + 1, 2, dtype=torch.float64, device=device) if sweep else None,
    )


def dspark_plan(B: int, gamma: int, kind: int, conf: torch.Tensor, sts_temp, min_verify_len: int,
                max_verify_len: int, survival_eps: float, budget_lo: int, budget_hi: int,
                cost_bias: float, cost_alpha: torch.Tensor, cost_theta: torch.Tensor,
                out: PlanOutputs, stream=None) -> PlanOutputs:
    f32, i32, f64 = torch.float32, torch.int32, torch.float64
    args = (
        B, gamma, kind,
        _ptr(conf, "conf", f32, B * gamma),
        _ptr(sts_temp, "sts_temp", f32, gamma, required=(kind == IN_CONF_LOGITS)),
        min_verify_len, max_verify_len, survival_eps, budget_lo, budget_hi, cost_bias,
        _ptr(cost_alpha, "cost_alpha", f32, 1), cost_alpha.numel(),
        _ptr(cost_theta, "cost_theta", f32, 1), cost_theta.numel(),
        _ptr(out.verify_lens, "verify_lens", i32, B),
        _ptr(out.plan_meta, "plan_meta", i32, 4),
        _ptr(out.plan_val, "plan_val", f64, 2),
        _ptr(out.survival_out, "survival_out", f32, B * gamma, required=False),
        _ptr(out.sweep_out, "sweep_out", f64, 2 * (B * gamma + 1), required=False),
        _stream(stream),
    )
    _lib.check("dspark_plan", _lib.lib().dspark_plan(*args))
    return out


# ------------------------------------------------------------------ pack

class PackOutputs(NamedTuple):
    cu_seqlens: torch.Tensor  # [B+1] int32
    packed_ids: torch.Tensor  # [capacity] int32
    packed_req: Optional[torch.Tensor]
    packed_pos: Optional[torch.Tensor]
    pack_meta: torch.Tensor  # [3] int32


def alloc_pack_outputs(B: int, capacity: int, device, req=True, pos=True) -> PackOutputs:
    i32 = torch.int32
    return PackOutputs(
        torch.empty(B + 1, dtype=i32, device=device),
        torch.empty(capacity, dtype=i32, device=device),
        torch.empty(capacity, dtype=i32, device=device) if req else None,
        torch.empty(capacity, dtype=i32, device=device) if pos else None,
        torch.empty(3, dtype=i32, device=device),
    )


def dspark_pack(B: int, gamma: int, verify_lens: torch.Tensor, anchor_ids: torch.Tensor,
                draft_tokens: torch.Tensor, tiers: Sequence[int], prefix_lens, out: PackOutputs,
                stream=None) -> PackOutputs:
    import ctypes

    i32 = torch.int32
    tiers = [int(t) for t in tiers]
    if not tiers:
        raise ValueError("tiers must not be empty")
    cap = tiers[-1]
    tiers_host = (ctypes.c_int32 * len(tiers))(*tiers)
    args = (
        B, gamma,
        _ptr(verify_lens, "verify_lens", i32, B),
        _ptr(anchor_ids, "anchor_ids", i32, B),
        _ptr(draft_tokens, "draft_tokens", i32, B * gamma),
        ctypes.cast(tiers_host, ctypes.c_void_p), len(tiers),
        _ptr(prefix_lens, "prefix_lens", i32, B, required=False),
        _ptr(out.cu_seqlens, "cu_seqlens", i32, B + 1),
        _ptr(out.packed_ids, "packed_ids", i32, cap),
        _ptr(out.packed_req, "packed_req", i32, cap, required=False),
        _ptr(out.packed_pos, "packed_pos", i32, cap, required=False),
        _ptr(out.pack_meta, "pack_meta", i32, 3),
        _stream(stream),
    )
    _lib.check("dspark_pack", _lib.lib().dspark_pack(*args))
    return out


def dspark_plan_pack(B: int, gamma: int, kind: int, conf: torch.Tensor, sts_temp,
                     min_verify_len: int, max_verify_len: int, survival_eps: float,
                     budget_lo: int, budget_hi: int, cost_bias: float, cost_alpha: torch.Tensor,
                     cost_theta: torch.Tensor, plan_out: PlanOutputs, anchor_ids: torch.Tensor,
                     draft_tokens: torch.Tensor, tiers: Sequence[int], prefix_lens,
                     pack_out: PackOutputs, stream=None):
    import ctypes

    f32, i32, f64 = torch.float32, torch.int32, torch.float64
    tiers = [int(t) for t in tiers]
    if not tiers:
        raise ValueError("tiers must not be empty")
    cap = tiers[-1]
    tiers_host = (ctypes.c_int32 * len(tiers))(*tiers)
    args = (
        B, gamma, kind,
        _ptr(conf, "conf", f32, B * gamma),
        _ptr(sts_temp, "sts_temp", f32, gamma, required=(kind == IN_CONF_LOGITS)),
        min_verify_len, max_verify_len, survival_eps, budget_lo, budget_hi, cost_bias,
        _ptr(cost_alpha, "cost_alpha", f32, 1), cost_alpha.numel(),
        _ptr(cost_theta, "cost_theta", f32, 1), cost_theta.numel(),
        _ptr(plan_out.verify_lens, "verify_lens", i32, B),
        _ptr(plan_out.plan_meta, "plan_meta", i32, 4),
        _ptr(plan_out.plan_val, "plan_val", f64, 2),
        _ptr(plan_out.survival_out, "survival_out", f32, B * gamma, required=False),
        _ptr(plan_out.sweep_out, "sweep_out", f64, 2 * (B * gamma + 1), required=False),
        _ptr(anchor_ids, "anchor_ids", i32, B),
        _ptr(draft_tokens, "draft_tokens", i32, B * gamma),
        ctypes.cast(tiers_host, ctypes.c_void_p), len(tiers),
        _ptr(prefix_lens, "prefix_lens", i32, B, required=False),
        _ptr(pack_out.cu_seqlens, "cu_seqlens", i32, B + 1),
        _ptr(pack_out.packed_ids, "packed_ids", i32, cap),
        _ptr(pack_out.packed_req, "packed_req", i32, cap, required=False),
        _ptr(pack_out.packed_pos, "packed_pos", i32, cap, required=False),
        _ptr(pack_out.pack_meta, "pack_meta", i32, 3),
        _stream(stream),
    )
    _lib.check("dspark_plan_pack", _lib.lib().dspark_plan_pack(*args))
    return plan_out, pack_out


def dspark_plan_pack_ex(B: int, gamma: int, kind: int, conf: torch.Tensor, sts_temp,
                        min_verify_len: int, max_verify_len: int, survival_eps: float,
                        budget_lo: int, budget_hi: int, cost_bias: float, cost_alpha,
                        cost_theta, plan_out: PlanOutputs, anchor_ids: torch.Tensor,
                        draft_tokens: torch.Tensor, tiers: Sequence[int], prefix_lens,
                        pack_out: PackOutputs, cost_mode: int = COST_ADDITIVE, sps_m=None,
                        sps=None, align_to_tier: bool = False, stream=None):
    """dspark_plan_pack with the 1D SPS cost model (``cost_mode=COST_SPS1D``,
    probe totals ``sps_m`` int32 and steps/s ``sps`` float32 on the device)
    and/or graph-tier alignment of the executed budget."""
    import ctypes

    f32, i32, f64 = torch.float32, torch.int32, torch.float64
    tiers = [int(t) for t in tiers]
    if not tiers:
        raise ValueError("tiers must not be empty")
    cap = tiers[-1]
    tiers_host = (ctypes.c_int32 * len(tiers))(*tiers)
    sps1d = cost_mode == COST_SPS1D
    n_probe = sps_m.numel() if sps1d else 0
    opt = _lib.PlanOptions(
        cost_mode,
        _ptr(sps_m, "sps_m", i32, n_probe, required=sps1d) if sps1d else None,
        _ptr(sps, "sps", f32, n_probe, required=sps1d) if sps1d else None,
        n_probe, 1 if align_to_tier else 0)
    args = (
        B, gamma, kind,
        _ptr(conf, "conf", f32, B * gamma),
        _ptr(sts_temp, "sts_temp", f32, gamma, required=(kind == IN_CONF_LOGITS)),
        min_verify_len, max_verify_len, survival_eps, budget_lo, budget_hi, cost_bias,
        _ptr(cost_alpha, "cost_alpha", f32, 1, required=not sps1d),
        cost_alpha.numel() if cost_alpha is not None else 0,
        _ptr(cost_theta, "cost_theta", f32, 1, required=not sps1d),
        cost_theta.numel() if cost_theta is not None else 0,
        _ptr(plan_out.verify_lens, "verify_lens", i32, B),
        _ptr(plan_out.plan_meta, "plan_meta", i32, 4),
        _ptr(plan_out.plan_val, "plan_val", f64, 2),
        _ptr(plan_out.survival_out, "survival_out", f32, B * gamma, required=False),
        _ptr(plan_out.sweep_out, "sweep_out", f64, 2 * (B * gamma + 1), required=False),
        _ptr(anchor_ids, "anchor_ids", i32, B),
        _ptr(draft_tokens, "draft_tokens", i32, B * gamma),
        ctypes.cast(tiers_host, ctypes.c_void_p), len(tiers),
        _ptr(prefix_lens, "prefix_lens", i32, B, required=False),
        _ptr(pack_out.cu_seqlens, "cu_seqlens", i32, B + 1),
        _ptr(pack_out.packed_ids, "packed_ids", i32, cap),
        _ptr(pack_out.packed_req, "packed_req", i32, cap, required=False),
        _ptr(pack_out.packed_pos, "packed_pos", i32, cap, required=False),
        _ptr(pack_out.pack_meta, "pack_meta", i32, 3),
        ctypes.cast(ctypes.pointer(opt), ctypes.c_void_p),
        _stream(stream),
    )
    _lib.check("dspark_plan_pack_ex", _lib.lib().dspark_plan_pack_ex(*args))
    return plan_out, pack_out


# ------------------------------------------------------------------ accept

class AcceptOutputs(NamedTuple):
    row_argmax: torch.Tensor  # [max_rows] int32
    num_correct: torch.Tensor  # [B] int32
    bonus: torch.Tensor
    commit_lens: torch.Tensor
    out_tokens: torch.Tensor  # [B, gamma+1] int32
    new_seq_lens: Optional[torch.Tensor]
    prefix_mask: Optional[torch.Tensor]  # [B, gamma] uint8
    accept_meta: torch.Tensor  # [2] int32
    workspace: torch.Tensor  # uint8 scratch (no initialization needed)


def dspark_accept_workspace_size(max_rows: int, V: int, dt: int) -> int:
    return int(_lib.lib().dspark_accept_workspace_size(max_rows, V, dt))


def alloc_accept_outputs(B: int, gamma: int, max_rows: int, V: int, dt: int, device,
                         new_seq=True, mask=True) -> AcceptOutputs:
    i32 = torch.int32
    ws = dspark_accept_workspace_size(max_rows, V, dt)
    return AcceptOutputs(
        torch.empty(max(max_rows, 1), dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, gamma + 1, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device) if new_seq else None,
        torch.empty(B, gamma, dtype=torch.uint8, device=device) if mask else None,
        torch.empty(2, dtype=i32, device=device),
        torch.empty(max(ws, 256), dtype=torch.uint8, device=device),
    )


def dspark_accept(B: int, gamma: int, V: int, dt: int, packed_logits: torch.Tensor, ld: int,
                  max_rows: int, cu_seqlens: torch.Tensor, draft_tokens: torch.Tensor,
                  prefix_lens, out: AcceptOutputs, stream=None) -> AcceptOutputs:
    i32 = torch.int32
    args = (
        B, gamma, V, dt,
        _ptr(packed_logits, "packed_logits", _logit_dtype(dt), max_rows * ld if max_rows else 0),
        ld, max_rows,
        _ptr(cu_seqlens, "cu_seqlens", i32, B + 1),
        _ptr(draft_tokens, "draft_tokens", i32, B * gamma),
        _ptr(prefix_lens, "prefix_lens", i32, B, required=False),
        _ptr(out.row_argmax, "row_argmax", i32, max_rows),
        _ptr(out.num_correct, "num_correct", i32, B),
        _ptr(out.bonus, "bonus", i32, B),
        _ptr(out.commit_lens, "commit_lens", i32, B),
        _ptr(out.out_tokens, "out_tokens", i32, B * (gamma + 1)),
        _ptr(out.new_seq_lens, "new_seq_lens", i32, B, required=False),
        _ptr(out.prefix_mask, "prefix_mask", torch.uint8, B * gamma, required=False),
        _ptr(out.accept_meta, "accept_meta", i32, 2),
        _ptr(out.workspace, "workspace", torch.uint8, 1), out.workspace.numel(),
        _stream(stream),
    )
    _lib.check("dspark_accept", _lib.lib().dspark_accept(*args))
    return out


NOALLOC_SCRATCH_BYTES = 1 << 20  # DSPARK_NOALLOC_SCRATCH_BYTES


def dspark_accept_noalloc(B: int, gamma: int, V: int, dt: int, packed_logits: torch.Tensor,
                          ld: int, max_rows: int, cu_seqlens: torch.Tensor,
                          draft_tokens: torch.Tensor, prefix_lens, out: AcceptOutputs,
                          stream=None) -> AcceptOutputs:
    """dspark_accept with the library's own scratch array instead of a
    workspace (out.workspace is not used); allocates nothing."""
    i32 = torch.int32
    args = (
        B, gamma, V, dt,
        _ptr(packed_logits, "packed_logits", _logit_dtype(dt), max_rows * ld if max_rows else 0),
        ld, max_rows,
        _ptr(cu_seqlens, "cu_seqlens", i32, B + 1),
        _ptr(draft_tokens, "draft_tokens", i32, B * gamma),
        _ptr(prefix_lens, "prefix_lens", i32, B, required=False),
        _ptr(out.row_argmax, "row_argmax", i32, max_rows),
        _ptr(out.num_correct, "num_correct", i32, B),
        _ptr(out.bonus, "bonus", i32, B),
        _ptr(out.commit_lens, "commit_lens", i32, B),
        _ptr(out.out_tokens, "out_tokens", i32, B * (gamma + 1)),
        _ptr(out.new_seq_lens, "new_seq_lens", i32, B, required=False),
        _ptr(out.prefix_mask, "prefix_mask", torch.uint8, B * gamma, required=False),
        _ptr(out.accept_meta, "accept_meta", i32, 2),
        _stream(stream),
    )
    _lib.check("dspark_accept_noalloc", _lib.lib().dspark_accept_noalloc(*args))
    return out


# ------------------------------------------------------------------ sampling accept

class SamplingOutputs(NamedTuple):
    num_correct: torch.Tensor  # [B] int32
    bonus: torch.Tensor  # [B] int32
    commit_lens: torch.Tensor  # [B] int32
    out_tokens: torch.Tensor  # [B, gamma+1] int32
    new_seq_lens: Optional[torch.Tensor]
    accept_meta: torch.Tensor  # [2] int32
    workspace: torch.Tensor  # uint8 scratch (no initialization needed)


def dspark_accept_sampling_workspace_size(B: int, gamma: int, V: int, dt: int) -> int:
    return int(_lib.lib().dspark_accept_sampling_workspace_size(B, gamma, V, dt))


def alloc_sampling_outputs(B: int, gamma: int, V: int, dt: int, device,
                           new_seq=True) -> SamplingOutputs:
    i32 = torch.int32
    ws = dspark_accept_sampling_workspace_size(B, gamma, V, dt)
    return SamplingOutputs(
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, gamma + 1, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device) if new_seq else None,
        torch.empty(2, dtype=i32, device=device),
        torch.empty(max(ws, 256), dtype=torch.uint8, device=device),
    )


def dspark_accept_sampling(B: int, gamma: int, V: int, dt: int, packed_logits: torch.Tensor,
                           ld: int, max_rows: int, cu_seqlens: torch.Tensor,
                           draft_logits: torch.Tensor, ld_q: int, draft_tokens: torch.Tensor,
                           temperatures: torch.Tensor, rand_accept: torch.Tensor,
                           rand_sample: torch.Tensor, prefix_lens, out: SamplingOutputs,
                           stream=None) -> SamplingOutputs:
    """Chain speculative-sampling accept. The random words are int32 tensors
    holding the uint32 bit patterns ([B, gamma] and [B, gamma + 1])."""
    i32 = torch.int32
    ldt = _logit_dtype(dt)
    args = (
        B, gamma, V, dt,
        _ptr(packed_logits, "packed_logits", ldt, max_rows * ld if max_rows else 0), ld, max_rows,
        _ptr(cu_seqlens, "cu_seqlens", i32, B + 1),
        _ptr(draft_logits, "draft_logits", ldt, (B * gamma - 1) * ld_q + V if B else 0), ld_q,
        _ptr(draft_tokens, "draft_tokens", i32, B * gamma),
        _ptr(temperatures, "temperatures", torch.float32, B),
        _ptr(rand_accept, "rand_accept", i32, B * gamma),
        _ptr(rand_sample, "rand_sample", i32, B * (gamma + 1)),
        _ptr(prefix_lens, "prefix_lens", i32, B, required=False),
        _ptr(out.num_correct, "num_correct", i32, B),
        _ptr(out.bonus, "bonus", i32, B),
        _ptr(out.commit_lens, "commit_lens", i32, B),
        _ptr(out.out_tokens, "out_tokens", i32, B * (gamma + 1)),
        _ptr(out.new_seq_lens, "new_seq_lens", i32, B, required=False),
        _ptr(out.accept_meta, "accept_meta", i32, 2),
        _ptr(out.workspace, "workspace", torch.uint8, 1), out.workspace.numel(),
        _stream(stream),
    )
    _lib.check("dspark_accept_sampling", _lib.lib().dspark_accept_sampling(*args))
    return out


# ------------------------------------------------------------------ cap-accept, scatter

class CapAcceptOutputs(NamedTuple):
    row_argmax: torch.Tensor  # [B * (gamma+1)] int32
    ceiling: torch.Tensor  # [B] int32
    num_correct: torch.Tensor  # [B] int32
    bonus: torch.Tensor
    commit_lens: torch.Tensor
    out_tokens: torch.Tensor  # [B, gamma+1] int32
    new_seq_lens: Optional[torch.Tensor]
    prefix_mask: Optional[torch.Tensor]  # [B, gamma] uint8
    accept_meta: torch.Tensor  # [2] int32
    workspace: torch.Tensor  # uint8 scratch (no initialization needed)


def alloc_cap_accept_outputs(B: int, gamma: int, V: int, dt: int, device, new_seq=True,
                             mask=True) -> CapAcceptOutputs:
    i32 = torch.int32
    rows = B * (gamma + 1)
    ws = dspark_accept_workspace_size(rows, V, dt)
    return CapAcceptOutputs(
        torch.empty(max(rows, 1), dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device),
        torch.empty(B, gamma + 1, dtype=i32, device=device),
        torch.empty(B, dtype=i32, device=device) if new_seq else None,
        torch.empty(B, gamma, dtype=torch.uint8, device=device) if mask else None,
        torch.empty(2, dtype=i32, device=device),
        torch.empty(max(ws, 256), dtype=torch.uint8, device=device),
    )


def dspark_cap_accept(B: int, gamma: int, V: int, dt: int, strided_logits: torch.Tensor, ld: int,
                      verify_lens: torch.Tensor, draft_tokens: torch.Tensor, prefix_lens,
                      out: CapAcceptOutputs, stream=None) -> CapAcceptOutputs:
    i32 = torch.int32
    rows = B * (gamma + 1)
    args = (
        B, gamma, V, dt,
        _ptr(strided_logits, "strided_logits", _logit_dtype(dt), rows * ld if rows else 0), ld,
        _ptr(verify_lens, "verify_lens", i32, B),
        _ptr(draft_tokens, "draft_tokens", i32, B * gamma),
        _ptr(prefix_lens, "prefix_lens", i32, B, required=False),
        _ptr(out.row_argmax, "row_argmax", i32, rows),
        _ptr(out.ceiling, "ceiling", i32, B),
        _ptr(out.num_correct, "num_correct", i32, B),
        _ptr(out.bonus, "bonus", i32, B),
        _ptr(out.commit_lens, "commit_lens", i32, B),
        _ptr(out.out_tokens, "out_tokens", i32, B * (gamma + 1)),
        _ptr(out.new_seq_lens, "new_seq_lens", i32, B, required=False),
        _ptr(out.prefix_mask, "prefix_mask", torch.uint8, B * gamma, required=False),
        _ptr(out.accept_meta, "accept_meta", i32, 2),
        _ptr(out.workspace, "workspace", torch.uint8, 1), out.workspace.numel(),
        _stream(stream),
    )
    _lib.check("dspark_cap_accept", _lib.lib().dspark_cap_accept(*args))
    return out


def dspark_scatter_to_strided(B: int, stride: int, cu_seqlens: torch.Tensor, packed: torch.Tensor,
                              strided: torch.Tensor, row_elems: int, scatter_meta: torch.Tensor,
                              stream=None) -> torch.Tensor:
    """Copy packed rows ``packed[cu[r] + j]`` to ``strided[r * stride + j]``.

    ``packed`` is [max_rows, ld_p] and ``strided`` [B * stride, ld_s], both 2-D,
    contiguous and of one element type; ``row_elems`` elements of each row are
    copied."""
    for name, t in (("packed", packed), ("strided", strided)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D torch.Tensor")
    if packed.dtype != strided.dtype:
        raise TypeError("packed and strided must share an element type")
    es = packed.element_size()
    max_rows = packed.shape[0]
    if strided.shape[0] < B * stride:
        raise ValueError(f"strided holds {strided.shape[0]} rows, needs {B * stride}")
    if row_elems > min(packed.shape[1], strided.shape[1]):
        raise ValueError("row_elems exceeds a row")
    args = (
        B, stride,
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, B + 1),
        max_rows,
        _ptr(packed, "packed", packed.dtype, 1 if max_rows else 0),
        packed.shape[1] * es,
        _ptr(strided, "strided", strided.dtype, 1 if B else 0),
        strided.shape[1] * es,
        row_elems * es,
        _ptr(scatter_meta, "scatter_meta", torch.int32, 2),
        _stream(stream),
    )
    _lib.check("dspark_scatter_to_strided", _lib.lib().dspark_scatter_to_strided(*args))
    return strided


# ------------------------------------------------------------------ STS fitter

class StsFit(NamedTuple):
    temps: torch.Tensor  # [gamma] float32
    t_index: torch.Tensor  # [gamma] int32
    ece: torch.Tensor  # [gamma] float64
    brier: torch.Tensor  # [gamma] float64
    ece_grid: Optional[torch.Tensor]  # [gamma, n_t] float64
    survival: Optional[torch.Tensor]  # [N, gamma] float32


def dspark_sts_workspace_size(N: int, gamma: int, n_t: int, n_bins: int) -> int:
    return int(_lib.lib().dspark_sts_workspace_size(N, gamma, n_t, n_bins))


def dspark_sts_fit(z: torch.Tensor, prefix_mask: torch.Tensor, t_grid: Sequence[float],
                   n_bins: int, survival=True, ece_grid=True, stream=None,
                   workspace: Optional[torch.Tensor] = None) -> StsFit:
    """Fit one STS temperature per position on records ``z`` [N, gamma] (float32
    confidence logits) and ``prefix_mask`` [N, gamma] (uint8 greedy labels).
    ``workspace`` (uint8, at least dspark_sts_workspace_size bytes) is
    allocated per call when not given."""
    import ctypes

    if z.dim() != 2:
        raise ValueError("z must be [N, gamma]")
    N, gamma = z.shape
    grid = [float(t) for t in t_grid]
    n_t = len(grid)
    grid_host = (ctypes.c_float * max(n_t, 1))(*grid)
    dev = z.device
    out = StsFit(
        torch.empty(gamma, dtype=torch.float32, device=dev),
        torch.empty(gamma, dtype=torch.int32, device=dev),
        torch.empty(gamma, dtype=torch.float64, device=dev),
        torch.empty(gamma, dtype=torch.float64, device=dev),
        torch.empty(gamma, max(n_t, 1), dtype=torch.float64, device=dev) if ece_grid else None,
        torch.empty(N, gamma, dtype=torch.float32, device=dev) if survival else None,
    )
    ws_bytes = dspark_sts_workspace_size(N, gamma, n_t, n_bins)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 256),
                                                             dtype=torch.uint8, device=dev)
    args = (
        N, gamma,
        _ptr(z, "z", torch.float32, N * gamma),
        _ptr(prefix_mask, "prefix_mask", torch.uint8, N * gamma),
        ctypes.cast(grid_host, ctypes.c_void_p), n_t, n_bins,
        _ptr(out.temps, "temps", torch.float32, gamma),
        _ptr(out.t_index, "t_index", torch.int32, gamma),
        _ptr(out.ece, "ece", torch.float64, gamma),
        _ptr(out.brier, "brier", torch.float64, gamma),
        _ptr(out.ece_grid, "ece_grid", torch.float64, gamma * n_t, required=False),
        _ptr(out.survival, "survival", torch.float32, N * gamma, required=False),
        _ptr(ws, "workspace", torch.uint8, 1), ws.numel(),
        _stream(stream),
    )
    _lib.check("dspark_sts_fit", _lib.lib().dspark_sts_fit(*args))
    return out


# ------------------------------------------------------------------ TV

def dspark_tv_accept(B: int, gamma: int, V: int, dt: int, draft_logits: torch.Tensor, ld_q: int,
                     target_logits: torch.Tensor, ld_p: int, target_rows_per_req: int,
                     accept_rate: torch.Tensor, survival: torch.Tensor, stream=None):
    ldt = _logit_dtype(dt)
    f32 = torch.float32
    args = (
        B, gamma, V, dt,
        _ptr(draft_logits, "draft_logits", ldt, (B * gamma - 1) * ld_q + V if B else 0), ld_q,
        _ptr(target_logits, "target_logits", ldt,
             ((B - 1) * target_rows_per_req + gamma - 1) * ld_p + V if B else 0), ld_p,
        target_rows_per_req,
        _ptr(accept_rate, "accept_rate", f32, B * gamma),
        _ptr(survival, "survival", f32, B * gamma),
        _stream(stream),
    )
    _lib.check("dspark_tv_accept", _lib.lib().dspark_tv_accept(*args))
    return accept_rate, survival
