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


def test_repad_hand_worked_example():
    """tests/golden/repad_example.json: three requests (one accepted draft plus the extra token, a
    K = 0 round, a rejected request) repadded to width 5, padding on either side."""
    g = json.load(open(os.path.join(GOLDEN, "repad_example.json")))
    for side, left in (("left_pad", True), ("right_pad", False)):
        res = C.repad(g["ragged_offsets"], g["accepted_len"], np.array(g["out_tokens"], dtype=np.int32),
                      g["prefix_offsets"], g["prefix_tokens"], g["width"], g["pad_id"], left)
        for key in ("token_ids", "position_ids", "mask", "row_len"):
            assert res[key].tolist() == g[side][key], (side, key)


def test_repad_invariants_on_oracle_verdicts():
    """Section 0x03C's position invariant (the unpadded positions of each row are 0 .. L - 1 and
    padding takes none), unpadding recovers the prefix followed by the packed commit's tokens, both
    padding sides hold the same sequence, and a row longer than the width is all padding."""
    rng = np.random.default_rng(11)
    depths = rng.integers(0, 9, size=90)
    b = make_random("repad", depths, 48, "fp32", 1.0, 2.0, 1.0, data_seed=11, verify_seed=12)
    stops = [list(rng.choice(48, size=rng.integers(0, 3), replace=False)) for _ in range(b.B)]
    budget = rng.integers(0, 8, size=b.B)
    v = oracle.verify(b.target, b.draft, b.tokens, b.cu, 1.0, 12, stop_lists=stops, budget=budget)
    plen = rng.integers(0, 20, size=b.B)
    po = np.concatenate([[0], np.cumsum(plen)])
    pt = rng.integers(0, 48, size=int(po[-1]))
    packed = C.commit(b.cu, v["accepted_len"], v["out_tokens"], plen, emitted_len=v["emitted_len"])
    width = int(np.max(packed["lengths"][:, 0])) - 3  # the longest rows do not fit
    sides = [C.repad(b.cu, v["accepted_len"], v["out_tokens"], po, pt, width, -7, left, v["emitted_len"])
             for left in (True, False)]
    for i in range(b.B):
        want = list(pt[po[i]:po[i + 1]]) + list(packed["tokens"][packed["offsets"][i]:packed["offsets"][i + 1]])
        L = len(want)
        assert L == packed["lengths"][i, 0]
        for res in sides:
            assert res["row_len"][i] == L
            keep = res["mask"][i].astype(bool)
            if L > width:
                assert not keep.any() and (res["token_ids"][i] == -7).all() and (res["position_ids"][i] == -1).all()
                continue
            assert res["token_ids"][i][keep].tolist() == want
            assert res["position_ids"][i][keep].tolist() == list(range(L))
            assert (res["token_ids"][i][~keep] == -7).all() and (res["position_ids"][i][~keep] == -1).all()
        if L <= width:
            assert sides[0]["mask"][i, width - L:].all() and sides[1]["mask"][i, :L].all()
    assert (sides[0]["row_len"] > width).any()


def test_repad_malformed_prefix_offsets_mark_their_row_alone():
    cu = offsets_from_depths([1, 1, 1])
    acc = np.array([0, 1, 0])
    out = np.array([3, -1, 4, 5, 6, -1], dtype=np.int32)
    res = C.repad(cu, acc, out, [0, 2, 1, 3], [9, 9, 9], 4, 0, True)
    assert res["row_len"].tolist() == [3, -1, 3]
    assert not res["mask"][1].any()
    assert res["token_ids"][0].tolist() == [0, 9, 9, 3] and res["token_ids"][2].tolist() == [0, 9, 9, 6]
