"""Pins for the layout (pack) and greedy-accept oracles.

Fixed by the pages' printed examples (golden fixtures): cu_seqlens of
[2,1,4]; the 7/12, 10/15 and 18/28 row counts; the tier roundings 37->40,
58->64, 65->80 and 63/64/65 -> 64/64/96; the A B C D vs A B X accept chain;
the all-accepted case; the prefix_mask of num_correct_drafts = 3; the
10 + 3 = 13 KV frontier; and the cap-accept counts [1,0,3]. Also fixed by
brute force and invariants: the first-index argmax with ties, NaN and signed
zeros against a pure-Python scan; static mode (every request verifies gamma+1
rows) against plain leading-match counting on the strided logits; and
sum(commit) = B + sum(correct).
"""

import numpy as np
import pytest

import oracle
from oracle.accept import as_f32_rows
from conftest import golden


def _tok(names):
    table = {}
    return [table.setdefault(n, 100 + len(table)) for n in names], table


def test_cu_seqlens_and_row_counts_from_pages():
    g = golden("layout_examples.json")
    for case in g["cases"]:
        lens = case["verify_lens"]
        B, gamma = len(lens), max(lens) - 1
        out = oracle.pack(B, gamma, lens, list(range(B)), np.zeros((B, gamma), np.int32),
                          [sum(lens)])
        cu = out["cu_seqlens"].tolist()
        assert cu[-1] == case["total"] == out["meta"][0]
        if "cu_seqlens" in case:
            assert cu == case["cu_seqlens"]
        if "strided_rows" in case:
            assert B * case["stride"] == case["strided_rows"]
        if "padded_rows" in case:
            assert B * max(lens) == case["padded_rows"]


def test_tier_rounding_from_pages():
    g = golden("tier_examples.json")
    for case in g["cases"]:
        total = case["total"]
        # one request per row keeps the total exact: B = total, all lengths 1
        out = oracle.pack(total, 1, [1] * total, list(range(total)), np.zeros((total, 1), np.int32),
                          case["tiers"])
        assert out["meta"][0] == total and out["meta"][1] == case["tier"]
        if "padding" in case:
            assert out["meta"][1] - out["meta"][0] == case["padding"]
            assert np.all(out["req"][total:] == -1) and np.all(out["ids"][total:] == 0)


def test_front_packing_rows():
    anchors = [7, 8, 9]
    drafts = np.array([[11, 12, 13], [21, 22, 23], [31, 32, 33]], np.int32)
    out = oracle.pack(3, 3, [2, 1, 4], anchors, drafts, [4, 8, 12], prefix_lens=[10, 20, 30])
    assert out["ids"].tolist() == [7, 11, 8, 9, 31, 32, 33, 0]
    assert out["req"].tolist() == [0, 0, 1, 2, 2, 2, 2, -1]
    assert out["pos"].tolist() == [10, 11, 20, 30, 31, 32, 33, 0]
    assert out["meta"].tolist() == [7, 8, 0]


def test_pack_flags_bad_lengths():
    out = oracle.pack(2, 2, [0, 5], [1, 2], np.zeros((2, 2), np.int32), [6])
    assert out["meta"][2] == oracle.DATA_BAD_LENS
    assert out["cu_seqlens"].tolist() == [0, 1, 4]  # clamped into [1, gamma + 1]


def _argmax_brute(row):
    """Pure-Python scan: first index of the maximum, NaN greatest, -0 == +0."""
    best = 0
    for i in range(1, len(row)):
        a, b = float(row[i]), float(row[best])
        if b != b:
            continue
        if a != a or a > b:
            best = i
    return best


def test_row_argmax_ties_nan_signed_zero():
    rows = np.array([
        [1.0, 3.0, 3.0, 2.0],
        [-0.0, 0.0, -1.0, -0.0],
        [0.0, -0.0, -1.0, 0.0],
        [1.0, np.nan, 5.0, np.nan],
        [-np.inf, -np.inf, -np.inf, -np.inf],
        [-5.0, -2.0, -2.0, -3.0],
        [np.inf, 1.0, np.inf, 0.0],
    ], dtype=np.float32)
    got = oracle.row_argmax(rows).tolist()
    assert got == [_argmax_brute(r) for r in rows] == [1, 0, 0, 1, 0, 1, 0]


@pytest.mark.parametrize("seed", range(5))
def test_row_argmax_random_bf16_against_scan(seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 16, size=(6, 300)).astype(np.uint16)  # includes NaNs and infs
    bits[:, 50] = bits[:, 10]  # force duplicates
    f = as_f32_rows(bits, "bf16")
    assert oracle.row_argmax(f).tolist() == [_argmax_brute(r) for r in f]


def _one_hot_rows(V, ids):
    rows = np.zeros((len(ids), V), dtype=np.float32)
    rows[np.arange(len(ids)), ids] = 1.0
    return rows


def test_accept_chain_examples_from_pages():
    g = golden("accept_examples.json")
    for case in g["cases"]:
        names = case["drafts"] + case["predictions"]
        _, table = _tok(names)
        d = [table[n] for n in case["drafts"]]
        pred = [table[n] for n in case["predictions"]]
        gamma = len(d)
        rows = _one_hot_rows(200, pred[: gamma + 1])
        out = oracle.accept(1, gamma, rows, "f32", [0, gamma + 1], np.array([d], np.int32),
                            prefix_lens=[g["frontier"]["prefix_len"]])
        assert out["num_correct"][0] == case["correct_len"]
        assert out["bonus"][0] == table[case["bonus"]]
        assert out["commit"][0] == case["commit_lens"]
        prefix = out["out_tokens"][0, : out["commit"][0]].tolist()
        assert prefix == [table[n] for n in case["output_prefix"]]
    fr = g["frontier"]
    # the first case commits 3 rows on a 10-token prefix -> 13
    names = ["A", "B", "C", "D", "X"]
    _, table = _tok(names)
    rows = _one_hot_rows(200, [table[n] for n in ["A", "B", "X", "D", "D"]])
    out = oracle.accept(1, 4, rows, "f32", [0, 5], np.array([[table[n] for n in "ABCD"]], np.int32),
                        prefix_lens=[fr["prefix_len"]])
    assert out["commit"][0] == fr["commit_lens"] and out["new_seq"][0] == fr["new_seq_len"]


def test_prefix_mask_example_from_pages():
    g = golden("prefix_mask_example.json")
    gamma = 6
    pred = [5, 6, 7, 99, 9, 10, 11]  # drafts match at 1..3, mismatch at 4, match again at 5
    drafts = np.array([[5, 6, 7, 8, 9, 10]], np.int32)
    out = oracle.accept(1, gamma, _one_hot_rows(128, pred), "f32", [0, gamma + 1], drafts)
    assert out["num_correct"][0] == g["num_correct_drafts"]
    assert out["prefix_mask"][0, :5].tolist() == g["prefix_mask_head"]


def test_cap_accept_counts_from_pages():
    g = golden("layout_examples.json")["cases"][0]
    lens = g["verify_lens"]
    B, N = len(lens), g["stride"]
    gamma = N - 1
    # every draft matches its target prediction
    drafts = np.arange(B * gamma, dtype=np.int32).reshape(B, gamma) + 1
    packed = oracle.pack(B, gamma, lens, [0] * B, drafts, [sum(lens)])
    preds = []
    for r in range(B):
        for j in range(lens[r]):
            preds.append(drafts[r, j] if j < gamma else 0)
    rows = _one_hot_rows(64, preds)
    out = oracle.accept(B, gamma, rows, "f32", packed["cu_seqlens"], drafts)
    assert out["num_correct"].tolist() == g["cap_accept_max_correct"]


@pytest.mark.parametrize("seed", range(6))
def test_static_mode_equals_plain_leading_match(seed):
    rng = np.random.default_rng(seed)
    B, gamma, V = 5, 6, 50
    logits = rng.normal(size=(B, gamma + 1, V)).astype(np.float32)
    am = logits.argmax(axis=2)
    drafts = np.where(rng.random((B, gamma)) < 0.7, am[:, :gamma], (am[:, :gamma] + 1) % V).astype(np.int32)
    cu = np.arange(B + 1) * (gamma + 1)
    out = oracle.accept(B, gamma, logits.reshape(-1, V), "f32", cu, drafts, prefix_lens=np.arange(B))
    for r in range(B):
        n = 0
        for k in range(gamma):
            if drafts[r, k] != am[r, k]:
                break
            n += 1
        assert out["num_correct"][r] == n and out["bonus"][r] == am[r, n]
        assert out["out_tokens"][r, :n].tolist() == drafts[r, :n].tolist()
        assert out["out_tokens"][r, n] == am[r, n]
    assert out["commit"].sum() == B + out["num_correct"].sum()
    assert np.array_equal(out["new_seq"], np.arange(B) + out["commit"])


def test_accept_flags_malformed_layout():
    rows = np.zeros((4, 8), np.float32)
    out = oracle.accept(2, 2, rows, "f32", [0, 3, 5], np.ones((2, 2), np.int32), max_rows=4)
    assert out["meta"].tolist() == [5, oracle.DATA_BAD_LENS]
    assert out["num_correct"][0] == 0 and out["commit"][0] == 1  # request 0 fits
    assert out["commit"][1] == 0 and out["bonus"][1] == -1  # request 1 overruns max_rows
    out = oracle.accept(2, 2, rows, "f32", [0, 0, 2], np.zeros((2, 2), np.int32))
    assert out["meta"][1] == oracle.DATA_BAD_LENS and out["commit"][0] == 0
