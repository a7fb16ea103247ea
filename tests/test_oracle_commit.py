"""Pins for the post-verification commit (oracle/commit.py): M7.8 section 0x09's worked example of
the lengths after a round (P = 10, K = 4), the position invariant of section 0x03C (each request's
new tokens sit at contiguous positions from its prefix length), and packing against numpy's cumsum
on verdicts produced by the oracle itself."""
import json
import os

import numpy as np

from oracle import commit as C
from oracle import oracle
from workloads import make_random, offsets_from_depths

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_m78_lengths_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "m78_stopping.json")))
    P, K = g["P"], g["K"]
    cu = offsets_from_depths([K])
    out = np.array([3, 8, 1, 12, 6], dtype=np.int32)  # all four drafts accepted, bonus 6
    for case, n_emit in zip(g["cases"], (4, 5, 5)):
        res = C.commit(cu, [K], out, [P], emitted_len=[n_emit])
        assert res["lengths"][0].tolist() == case["expect"], case["what"]
        assert res["tokens"].tolist() == out[:n_emit].tolist()
        assert res["positions"].tolist() == list(range(P, P + n_emit))


def test_position_invariant_and_packing_on_oracle_verdicts():
    rng = np.random.default_rng(3)
    depths = rng.integers(0, 9, size=120)
    b = make_random("commit", depths, 64, "fp32", 1.0, 2.0, 1.0, data_seed=3, verify_seed=4)
    stops = [list(rng.choice(64, size=rng.integers(0, 3), replace=False)) for _ in range(b.B)]
    budget = rng.integers(0, 8, size=b.B)
    v = oracle.verify(b.target, b.draft, b.tokens, b.cu, 1.0, 4, stop_lists=stops, budget=budget)
    prefix = rng.integers(0, 1000, size=b.B)
    res = C.commit(b.cu, v["accepted_len"], v["out_tokens"], prefix, emitted_len=v["emitted_len"])
    n = v["emitted_len"].astype(np.int64)
    assert np.array_equal(res["offsets"], np.concatenate([[0], np.cumsum(n)]))
    for i in range(b.B):
        seg = slice(res["offsets"][i], res["offsets"][i + 1])
        assert np.array_equal(res["positions"][seg], prefix[i] + np.arange(n[i]))
        slots = v["out_tokens"][b.cu[i] + i: b.cu[i + 1] + i + 1]
        assert np.array_equal(res["tokens"][seg], slots[:n[i]])
        assert res["lengths"][i, 0] == prefix[i] + n[i]  # L_out = P + E + F = P + emitted
        if n[i]:
            assert res["next_token"][i] == slots[n[i] - 1] and res["next_position"][i] == prefix[i] + n[i] - 1
        else:
            assert res["next_token"][i] == -1


def test_without_emitted_len_every_valid_request_emits_a_plus_one():
    cu = offsets_from_depths([2, 0, 3])
    acc = np.array([1, 0, -1])
    out = np.array([5, 7, -1, 9, -1, -1, -1, -1], dtype=np.int32)
    res = C.commit(cu, acc, out, [0, 4, 9])
    assert res["offsets"].tolist() == [0, 2, 3, 3]
    assert res["tokens"].tolist() == [5, 7, 9]
    assert res["positions"].tolist() == [0, 1, 4]
    assert res["lengths"].tolist() == [[2, 1, 1], [5, 4, 4], [9, 9, 9]]
