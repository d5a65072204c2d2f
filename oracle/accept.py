"""Greedy accept oracle: row argmax, leading-match count, bonus, finalize.

Test infrastructure only (see ``oracle/__init__.py``).

* ``target_predict = argmax(target_logits)`` per packed row ([Round] §五,
  AcceptGreedy; [Budget] §二, the STS recorder). Ties go to the lowest
  index. Values compare as float32 after exact widening of bfloat16. -0
  equals +0, and NaN ranks above every number (the first NaN wins).
* Draft position k is checked against the prediction of verify row k-1
  (row 0 is the root): the prediction of R checks A, that of A checks B
  ([Round] §四). ``correct`` counts the leading matches, at most
  ``verify_len - 1``, and stops at the first mismatch: a later isolated match
  is not accepted ([Budget] §二, the prefix_mask example; [CSSD], prefix
  event).
* ``bonus`` is the prediction of the last valid input row, ``am[cu[r] +
  correct]`` ([Round] §五).
* FinalizeAcceptLens: ``commit = correct + 1`` and
  ``new_seq = prefix + commit`` ([Round] §五 and §六; [Budget] §三).
* BuildOutTokens: ``out[:, :gamma] = drafts``, then ``bonus`` is scattered at
  column ``correct`` ([Round] §五). Column gamma starts at -1 (reading: the
  buffer's initial value is unspecified).
* ``prefix_mask[r, k-1] = (k <= correct)`` ([Budget] §二).
* Reading for malformed layouts: a request whose rows are not
  ``1..gamma+1`` rows inside ``[0, min(cu[B], max_rows))`` sets
  DATA_BAD_LENS. Its outputs are correct 0, bonus -1, commit 0,
  out_tokens -1, prefix_mask 0 and new_seq = prefix.
"""

from __future__ import annotations

import numpy as np

from .pack import DATA_BAD_LENS


def as_f32_rows(rows, dtype: str) -> np.ndarray:
    """float32 view of logit rows given as float32 or as bfloat16 bit patterns."""
    if dtype == "bf16":
        return (np.asarray(rows, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(rows, dtype=np.float32)


def row_argmax(rows_f32: np.ndarray) -> np.ndarray:
    """First index of the row maximum (NaN greatest, -0 == +0).

    ``numpy.argmax`` returns the first occurrence of the maximum, and returns the
    first NaN when a row holds one. -0 and +0 compare equal."""
    rows_f32 = np.asarray(rows_f32, dtype=np.float32)
    if rows_f32.shape[0] == 0:
        return np.zeros(0, dtype=np.int32)
    return np.argmax(rows_f32, axis=1).astype(np.int32)


def accept(B, gamma, rows, dtype, cu_seqlens, drafts, prefix_lens=None, max_rows=None,
           row_am=None):
    """Greedy accept over packed logit rows ``rows[max_rows, V]``.

    ``row_am`` may pass precomputed row argmaxes (from this module) to skip
    the vocab pass. Returns a dict with ``row_argmax`` (rows ``< total``),
    ``num_correct``, ``bonus``, ``commit``, ``new_seq``, ``out_tokens``,
    ``prefix_mask`` and ``meta`` = (cu[B], status)."""
    B, gamma = int(B), int(gamma)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if max_rows is None:
        max_rows = rows.shape[0]
    total = int(cu[B])
    total_eff = min(max(total, 0), int(max_rows))
    status = 0 if total == total_eff else DATA_BAD_LENS
    am = row_argmax(as_f32_rows(rows[:total_eff], dtype)) if row_am is None else np.asarray(row_am)

    num_correct = np.zeros(B, dtype=np.int32)
    bonus = np.full(B, -1, dtype=np.int32)
    commit = np.zeros(B, dtype=np.int32)
    prefix = np.zeros(B, dtype=np.int64) if prefix_lens is None else np.asarray(prefix_lens, dtype=np.int64)
    new_seq = prefix.astype(np.int32).copy()
    out = np.full((B, gamma + 1), -1, dtype=np.int32)
    mask = np.zeros((B, gamma), dtype=np.uint8)
    for r in range(B):
        a, e = int(cu[r]), int(cu[r + 1])
        length = e - a
        if not (a >= 0 and 1 <= length <= gamma + 1 and e <= total_eff):
            status |= DATA_BAD_LENS
            continue
        c = 0
        while c < length - 1 and int(drafts[r][c]) == int(am[a + c]):
            c += 1
        num_correct[r] = c
        bonus[r] = am[a + c]
        commit[r] = c + 1
        new_seq[r] = prefix[r] + c + 1
        out[r, :gamma] = drafts[r]
        out[r, c] = am[a + c]
        mask[r, :c] = 1
    return {"row_argmax": am[:total_eff].astype(np.int32), "num_correct": num_correct,
            "bonus": bonus, "commit": commit, "new_seq": new_seq, "out_tokens": out,
            "prefix_mask": mask, "meta": np.array([total, status], dtype=np.int32)}
