"""Compact ragged layout oracle: cu_seqlens, front-packing, tier rounding.

Test infrastructure only (see ``oracle/__init__.py``).

* ``cu_seqlens`` is the exclusive prefix sum of ``verify_lens`` with a
  leading 0 ([Budget] §六, ``cu_seqlens_q = [0,2,3,7]`` for lengths
  ``[2,1,4]``).
* Each request's rows are front-packed back to back: row 0 is the root
  (anchor) token, row j >= 1 is draft j ([Round] §三: ``verify_ids_2d`` is
  the anchor followed by the drafts, and compact mode packs the anchor plus
  the selected draft prefix; [Budget] §五, the ``A0 A1 | B0 | C0..C3``
  example).
* The packed total is rounded up to the smallest captured tier that holds it
  ([SGLang], ragged verify; [CSSD], graph tiers: 37 -> 40, 58 -> 64,
  65 -> 80).
* Reading for the unspecified parts: pad rows ``[total, tier)`` get id 0,
  request -1 and position 0. The position of row j is
  ``prefix_len[r] + j`` ([Round] §六: the anchor sits at the old KV
  frontier), or j when no prefix lengths are given. A length outside
  ``[1, gamma + 1]`` sets DATA_BAD_LENS and is clamped into that range
  before packing.
"""

from __future__ import annotations

import numpy as np

DATA_BAD_LENS = 4


def pack(B, gamma, verify_lens, anchors, drafts, tiers, prefix_lens=None):
    """Returns dict: ``cu_seqlens`` int32[B+1]; ``ids``, ``req``, ``pos``
    int32[tier]; ``meta`` int32[3] = (total, tier, status)."""
    B, gamma = int(B), int(gamma)
    status = 0
    lens = []
    for r in range(B):
        length = int(verify_lens[r])
        if not (1 <= length <= gamma + 1):
            status |= DATA_BAD_LENS
            length = min(max(length, 1), gamma + 1)
        lens.append(length)
    cu = [0]
    for length in lens:
        cu.append(cu[-1] + length)
    total = cu[-1]
    tier = next(int(t) for t in tiers if int(t) >= total)
    ids = np.zeros(tier, dtype=np.int32)
    req = np.full(tier, -1, dtype=np.int32)
    pos = np.zeros(tier, dtype=np.int32)
    for r in range(B):
        for j in range(lens[r]):
            i = cu[r] + j
            ids[i] = anchors[r] if j == 0 else drafts[r][j - 1]
            req[i] = r
            pos[i] = (int(prefix_lens[r]) if prefix_lens is not None else 0) + j
    return {"cu_seqlens": np.asarray(cu, dtype=np.int32), "ids": ids, "req": req, "pos": pos,
            "meta": np.array([total, tier, status], dtype=np.int32)}
