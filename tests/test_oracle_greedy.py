"""Pins for the oracle's Rule 1 (greedy) path.

"Speculative Decoding Coordination Protocol (SDCP)", section "Acceptance Rules", Rule 1: accept
x[i] iff it is the argmax of p[i] (smallest id on ties), stop at the first miss, emit the argmax of
the next row; the output equals greedy decoding of the target whatever the drafter proposes.
Section "Test Vectors" prints one worked round, stored in tests/golden/sdcp_greedy_round.json.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle
from workloads import bf16_bits, bf16_to_f32, offsets_from_depths

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "sdcp_greedy_round.json")


def _rows_with_argmax(argmaxes, V=16, seed=0, dtype="fp32"):
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((len(argmaxes), V)).astype(np.float32)
    for r, a in enumerate(argmaxes):
        rows[r, a] = rows[r].max() + 2.0
    return bf16_bits(rows) if dtype == "bf16" else rows


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sdcp_worked_round(dtype):
    g = json.load(open(GOLDEN))
    target = _rows_with_argmax(g["target_argmax"], dtype=dtype)
    tokens = np.array(g["proposal"], dtype=np.int32)
    cu = offsets_from_depths([len(tokens)])
    res = oracle.verify(target, None, tokens, cu, 0.0, seed=0)
    a = int(res["accepted_len"][0])
    assert a == g["expected_accepted"]
    assert res["out_tokens"][: a + 1].tolist() == g["expected_emitted"]
    assert res["out_tokens"][a + 1:].tolist() == [-1] * (len(tokens) - a)


def test_sdcp_worked_round_all_accepted_variant():
    g = json.load(open(GOLDEN))
    target = _rows_with_argmax(g["target_argmax"])
    tokens = np.array([7, 9, 13], dtype=np.int32)
    res = oracle.verify(target, None, tokens, offsets_from_depths([3]), 0.0, seed=0)
    assert res["accepted_len"].tolist() == [3]
    assert res["out_tokens"].tolist() == [7, 9, 13, 5]


def test_greedy_output_is_target_greedy_decoding_for_any_draft():
    rng = np.random.default_rng(7)
    V = 50
    depths = rng.integers(0, 9, size=40)
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    target = bf16_bits(rng.standard_normal((n_d + 40, V)).astype(np.float32) * 2)
    tv = bf16_to_f32(target)
    argm = np.argmax(tv, axis=1)
    for trial in range(20):
        # drafts agree with the target argmax with probability 0.7, else a random token
        t_of_d = np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(40)]).astype(int)
        agree = rng.random(n_d) < 0.7
        tokens = np.where(agree, argm[t_of_d], rng.integers(0, V, size=n_d)).astype(np.int32)
        res = oracle.verify(target, None, tokens, cu, 0.0, seed=trial)
        for i in range(40):
            K, base = int(depths[i]), int(cu[i] + i)
            a = int(res["accepted_len"][i])
            emitted = res["out_tokens"][base: base + a + 1]
            assert emitted.tolist() == argm[base: base + a + 1].tolist()
            drafted = tokens[cu[i]: cu[i + 1]]
            mism = np.nonzero(drafted != argm[base: base + K])[0]
            assert a == (int(mism[0]) if mism.size else K)
            assert (res["out_tokens"][base + a + 1: base + K + 1] == -1).all()


def test_greedy_ignores_draft_logits_and_seed():
    rng = np.random.default_rng(1)
    target = rng.standard_normal((5, 30)).astype(np.float32)
    draft = rng.standard_normal((4, 30)).astype(np.float32)
    tokens = np.argmax(target[:4], axis=1).astype(np.int32)
    cu = offsets_from_depths([4])
    a = oracle.verify(target, None, tokens, cu, 0.0, seed=1)
    b = oracle.verify(target, draft, tokens, cu, 0.0, seed=99)
    assert a["out_tokens"].tolist() == b["out_tokens"].tolist() == tokens.tolist() + [int(np.argmax(target[4]))]


def test_greedy_tie_goes_to_smallest_id():
    row = np.zeros((2, 10), dtype=np.float32)
    row[0, [3, 6]] = 5.0
    row[1, [0, 9]] = 1.0
    # proposing the larger tied id is a miss; the correction is the smaller one
    res = oracle.verify(row, None, np.array([6], dtype=np.int32), offsets_from_depths([1]), 0.0, seed=0)
    assert res["accepted_len"].tolist() == [0] and res["out_tokens"].tolist() == [3, -1]
    res = oracle.verify(row, None, np.array([3], dtype=np.int32), offsets_from_depths([1]), 0.0, seed=0)
    assert res["accepted_len"].tolist() == [1] and res["out_tokens"].tolist() == [3, 0]


def test_greedy_bad_tokens_reject_the_request_only():
    rng = np.random.default_rng(2)
    target = rng.standard_normal((3 + 2, 12)).astype(np.float32)
    tokens = np.array([1, 12, 4], dtype=np.int32)  # 12 is out of range for request 0
    res = oracle.verify(target, None, tokens, offsets_from_depths([2, 1]), 0.0, seed=0)
    assert res["accepted_len"][0] == -1 and res["out_tokens"][:3].tolist() == [-1, -1, -1]
    assert res["accepted_len"][1] in (0, 1)
