"""Pins for the strided-layout oracles (cap-accept, scatter to stride).

Fixed by the pages: the cap-accept example (lengths [2,1,4] at width 4 with
every draft matching: acceptable drafts [1,0,3] while the target runs 12
rows), the statement that cap-accept commits exactly what compact mode
commits, and the [2,5,3] stride-5 layout (10 of 15 strided rows hold
results). Also fixed by reduction to the already pinned accept oracle: the
ceiling equals static-mode accept (full verification) on the same rows, and
a scatter followed by reading the valid rows back is the identity.
"""

import numpy as np
import pytest

import oracle
from conftest import golden


def _one_hot_rows(V, ids):
    rows = np.zeros((len(ids), V), dtype=np.float32)
    rows[np.arange(len(ids)), ids] = 1.0
    return rows


def _strided_case(rng, B, gamma, V, p_match):
    """Strided logits, drafts that copy the row argmax with probability p_match."""
    logits = rng.normal(size=(B, gamma + 1, V)).astype(np.float32)
    am = logits.argmax(axis=2)
    hit = rng.random((B, gamma)) < p_match
    drafts = np.where(hit, am[:, :gamma], (am[:, :gamma] + 1 + rng.integers(0, V - 1, (B, gamma))) % V)
    return logits, drafts.astype(np.int32)


def test_cap_accept_counts_from_pages():
    g = golden("layout_examples.json")["cases"][0]
    lens = g["verify_lens"]
    B, width = len(lens), g["stride"]
    gamma = width - 1
    drafts = np.arange(B * gamma, dtype=np.int32).reshape(B, gamma) + 1
    preds = [int(drafts[r, j]) if j < gamma else 0 for r in range(B) for j in range(width)]
    rows = _one_hot_rows(64, preds)
    out = oracle.cap_accept(B, gamma, rows, "f32", lens, drafts)
    assert out["meta"].tolist() == [g["strided_rows"], 0]  # the target still runs 12 rows
    assert out["num_correct"].tolist() == g["cap_accept_max_correct"]
    assert out["ceiling"].tolist() == [gamma] * B
    assert out["commit"].tolist() == [c + 1 for c in g["cap_accept_max_correct"]]


@pytest.mark.parametrize("seed", range(8))
def test_cap_accept_commits_what_compact_commits(seed):
    rng = np.random.default_rng(100 + seed)
    B, gamma, V = 7, 5, 40
    logits, drafts = _strided_case(rng, B, gamma, V, 0.75)
    lens = rng.integers(1, gamma + 2, size=B).astype(np.int32)
    prefix = rng.integers(0, 50, size=B)
    cap = oracle.cap_accept(B, gamma, logits.reshape(-1, V), "f32", lens, drafts, prefix)
    cu = np.concatenate([[0], np.cumsum(lens)])
    packed = np.concatenate([logits[r, : lens[r]] for r in range(B)])
    comp = oracle.accept(B, gamma, packed, "f32", cu, drafts, prefix)
    for k in ("num_correct", "bonus", "commit", "new_seq", "out_tokens", "prefix_mask"):
        assert np.array_equal(cap[k], comp[k]), k
    valid = np.concatenate([np.arange(lens[r]) + r * (gamma + 1) for r in range(B)])
    assert np.array_equal(cap["row_argmax"][valid], comp["row_argmax"])
    assert np.all(cap["ceiling"] >= cap["num_correct"])


@pytest.mark.parametrize("seed", range(4))
def test_ceiling_is_static_mode_accept(seed):
    rng = np.random.default_rng(200 + seed)
    B, gamma, V = 6, 7, 30
    logits, drafts = _strided_case(rng, B, gamma, V, 0.85)
    lens = rng.integers(1, gamma + 2, size=B)
    cap = oracle.cap_accept(B, gamma, logits.reshape(-1, V), "f32", lens, drafts)
    full = oracle.accept(B, gamma, logits.reshape(-1, V), "f32", np.arange(B + 1) * (gamma + 1), drafts)
    assert np.array_equal(cap["ceiling"], full["num_correct"])
    assert np.array_equal(cap["row_argmax"], full["row_argmax"])


def test_trimming_hides_the_ceiling():
    B, gamma, V = 2, 4, 16
    drafts = np.array([[3, 4, 5, 6], [7, 8, 9, 10]], dtype=np.int32)
    preds = [3, 4, 5, 6, 11, 7, 8, 1, 1, 1]  # request 0 all match, request 1 two match
    rows = _one_hot_rows(V, preds)
    out = oracle.cap_accept(B, gamma, rows, "f32", [1, 5], drafts)
    assert out["ceiling"].tolist() == [4, 2]
    assert out["num_correct"].tolist() == [0, 2]
    assert out["bonus"].tolist() == [3, 1]  # row 0 of request 0 predicts draft 1
    assert out["out_tokens"].tolist() == [[3, 4, 5, 6, -1], [7, 8, 1, 10, -1]]


def test_cap_accept_flags_bad_lengths():
    B, gamma, V = 3, 2, 8
    rows = _one_hot_rows(V, [1, 2, 3] * B)
    drafts = np.array([[1, 2]] * B, dtype=np.int32)
    out = oracle.cap_accept(B, gamma, rows, "f32", [0, 3, 4], drafts, [5, 6, 7])
    assert out["meta"].tolist() == [B * (gamma + 1), oracle.DATA_BAD_LENS]
    assert out["ceiling"].tolist() == [2, 2, 2]
    assert out["num_correct"].tolist() == [0, 2, 0]
    assert out["bonus"].tolist() == [-1, 3, -1]
    assert out["commit"].tolist() == [0, 3, 0]
    assert out["new_seq"].tolist() == [5, 9, 7]
    assert out["out_tokens"][0].tolist() == [-1, -1, -1]
    assert out["prefix_mask"][2].tolist() == [0, 0]


def test_scatter_rows_from_pages():
    g = golden("layout_examples.json")["cases"][1]
    lens, stride = g["verify_lens"], g["stride"]
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    packed = np.arange(g["total"] * 3, dtype=np.int32).reshape(-1, 3) + 1000
    init = np.full((B * stride, 3), -7, dtype=np.int32)
    out, meta = oracle.scatter_to_strided(B, stride, cu, packed, init)
    assert meta.tolist() == [10, 0]
    written = [r * stride + j for r in range(B) for j in range(lens[r])]
    assert written == [0, 1, 5, 6, 7, 8, 9, 10, 11, 12]
    assert np.array_equal(out[written], packed)
    untouched = sorted(set(range(B * stride)) - set(written))
    assert len(untouched) == g["strided_rows"] - g["total"]
    assert np.all(out[untouched] == -7)


@pytest.mark.parametrize("seed", range(5))
def test_scatter_round_trip(seed):
    rng = np.random.default_rng(300 + seed)
    B, stride, D = 9, 6, 5
    strided = rng.normal(size=(B * stride, D)).astype(np.float32)
    lens = rng.integers(1, stride + 1, size=B)
    cu = np.concatenate([[0], np.cumsum(lens)])
    valid = np.concatenate([np.arange(lens[r]) + r * stride for r in range(B)])
    packed = np.concatenate([strided[valid], np.zeros((3, D), np.float32)])  # + pad rows
    init = np.full_like(strided, np.nan)
    out, meta = oracle.scatter_to_strided(B, stride, cu, packed, init, max_rows=packed.shape[0])
    assert meta.tolist() == [int(cu[-1]), 0]
    assert np.array_equal(out[valid], strided[valid])
    rest = np.setdiff1d(np.arange(B * stride), valid)
    assert np.all(np.isnan(out[rest]))


def test_scatter_flags_malformed_layouts():
    packed = np.arange(12, dtype=np.int32).reshape(6, 2)
    init = np.full((8, 2), -1, dtype=np.int32)
    # request 1 is empty, request 2 is longer than the stride, request 3 runs past max_rows
    out, meta = oracle.scatter_to_strided(4, 2, [0, 2, 2, 5, 7], packed, init, max_rows=6)
    assert meta.tolist() == [7, oracle.DATA_BAD_LENS]
    assert out[:2].tolist() == [[0, 1], [2, 3]]
    assert np.all(out[2:] == -1)
