"""Strided-layout oracles: cap-accept and the scatter of packed rows back to stride.

Test infrastructure only (see ``oracle/__init__.py``).

Cap-accept ([SGLang] "三种 verify mode" and "可观测性"; [CSSD] "static、
compact 与 cap-accept 三种模式"; [Budget] §五 cap-accept): the target still
runs the full block of gamma + 1 rows per request, in the fixed strided
layout, and only the accept step is limited by the planner's verify_lens.
``correct_len`` is clipped to ``verify_len - 1`` (for lens [2, 1, 4] with
width 4 and every draft matching, the acceptable drafts are [1, 0, 3]). The
committed result equals the compact mode's, and the uncapped count over the
full block, the acceptance ceiling that trimming hides, is reported beside
it.

Scatter ([Round] §三, ScatterCompactToStrided): after the forward pass on
the packed rows, each request's rows are copied back to the uniform
``[B, stride]`` logical layout, so that later stages address them by fixed
position. Rows past a request's verify length are not written: they were
never computed, and verify_lens still says which results are valid.

Readings (also in the design notes):

* Cap-accept's bonus is the prediction of row ``correct`` of the request
  (the same row compact mode reads), and the ceiling counts the leading
  matches of all gamma drafts against rows 0..gamma-1.
* A verify length outside ``[1, gamma + 1]`` sets DATA_BAD_LENS and gives
  that request the malformed-layout outputs of the compact accept (correct
  0, bonus -1, commit 0, out_tokens -1, mask 0, new_seq = prefix). Its
  ceiling is still reported: it does not depend on the length.
* Scatter: a request whose packed rows are not ``1..stride`` rows inside
  ``[0, min(cu[B], max_rows))`` sets DATA_BAD_LENS and none of its rows is
  written. The status also flags ``cu[B] > max_rows``.
"""

from __future__ import annotations

import numpy as np

from .accept import as_f32_rows, row_argmax
from .pack import DATA_BAD_LENS


def cap_accept(B, gamma, rows, dtype, verify_lens, drafts, prefix_lens=None):
    """Greedy accept over strided rows ``rows[B * (gamma + 1), V]`` capped by
    ``verify_lens``. Returns a dict with ``row_argmax`` (all strided rows),
    ``ceiling``, ``num_correct``, ``bonus``, ``commit``, ``new_seq``,
    ``out_tokens``, ``prefix_mask`` and ``meta`` = (rows, status)."""
    B, gamma = int(B), int(gamma)
    width = gamma + 1
    n_rows = B * width
    am = row_argmax(as_f32_rows(rows[:n_rows], dtype))
    prefix = np.zeros(B, dtype=np.int64) if prefix_lens is None else np.asarray(prefix_lens, dtype=np.int64)
    status = 0
    ceiling = np.zeros(B, dtype=np.int32)
    num_correct = np.zeros(B, dtype=np.int32)
    bonus = np.full(B, -1, dtype=np.int32)
    commit = np.zeros(B, dtype=np.int32)
    new_seq = prefix.astype(np.int32).copy()
    out = np.full((B, width), -1, dtype=np.int32)
    mask = np.zeros((B, gamma), dtype=np.uint8)
    for r in range(B):
        base = r * width
        # full block: draft k (column k-1) against the prediction of row k-1
        full = 0
        while full < gamma and int(drafts[r][full]) == int(am[base + full]):
            full += 1
        ceiling[r] = full
        length = int(verify_lens[r])
        if not 1 <= length <= width:
            status |= DATA_BAD_LENS
            continue
        c = min(full, length - 1)
        num_correct[r] = c
        bonus[r] = am[base + c]
        commit[r] = c + 1
        new_seq[r] = prefix[r] + c + 1
        out[r, :gamma] = drafts[r]
        out[r, c] = am[base + c]
        mask[r, :c] = 1
    return {"row_argmax": am.astype(np.int32), "ceiling": ceiling, "num_correct": num_correct,
            "bonus": bonus, "commit": commit, "new_seq": new_seq, "out_tokens": out,
            "prefix_mask": mask, "meta": np.array([n_rows, status], dtype=np.int32)}


def scatter_to_strided(B, stride, cu_seqlens, packed, strided_init, max_rows=None):
    """Copy packed rows ``packed[i]`` to ``strided[r * stride + j]`` for
    ``i = cu[r] + j``, ``j < cu[r+1] - cu[r]``. ``strided_init`` holds the
    destination's previous contents (rows that are not written keep them).
    Returns (strided, meta) with meta = (cu[B], status)."""
    B, stride = int(B), int(stride)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if max_rows is None:
        max_rows = packed.shape[0]
    total = int(cu[B])
    total_eff = min(max(total, 0), int(max_rows))
    status = 0 if total == total_eff else DATA_BAD_LENS
    out = np.array(strided_init, copy=True)
    for r in range(B):
        a, e = int(cu[r]), int(cu[r + 1])
        length = e - a
        if not (a >= 0 and 1 <= length <= stride and e <= total_eff):
            status |= DATA_BAD_LENS
            continue
        for j in range(length):
            out[r * stride + j] = packed[a + j]
    return out, np.array([total, status], dtype=np.int32)
