"""Pins for the oracle's verdict completion: stop tokens, the output budget, and caller-supplied
uniforms.

What fixes the answer:
  * M7.8 section 0x09's worked example of stopping (P = 10, K = 4: a length cap at draft_4 gives
    (L_out, L_target, L_draft) = (14, 14, 13), a cap or EOS at the bonus (15, 14, 13)), stored in
    tests/golden/m78_stopping.json;
  * SDCP's example round under the greedy rule with stop tokens and budgets (SDCP "Verification and
    Commit", step 7), tests/golden/sdcp_greedy_round_stops.json;
  * invariants: truncation never changes the accepted count nor which uniforms are used, so the
    emitted tokens are a prefix of the untruncated emission;
  * with the caller's uniforms, SDCP Rule 2's strict test r < p/q: r = 0 accepts every draft whose
    target probability is positive and rejects one whose target probability is zero; a request
    with no drafts draws its token with numpy's searchsorted on the CDF at the caller's u; and
    uniform r, u drawn from numpy make the output follow the exact law (enumeration).
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import exact, oracle
from workloads import make_random, offsets_from_depths

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _greedy_rows(argmaxes, V=16, seed=0):
    """Target rows whose argmax is the given token (distinct maxima)."""
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((len(argmaxes), V)).astype(np.float32)
    for r, g in enumerate(argmaxes):
        rows[r, g] = rows[r].max() + 1.0
    return rows


def test_m78_stopping_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "m78_stopping.json")))
    P, K = g["P"], g["K"]
    drafts = [3, 8, 1, 12]
    bonus = 6
    target = _greedy_rows(drafts + [bonus])
    for case in g["cases"]:
        stops = [[bonus]] if case["stop_at_bonus"] else [[]]
        budget = [case["budget"]] if case["budget"] is not None else None
        res = oracle.verify(target, None, np.array(drafts, dtype=np.int32), offsets_from_depths([K]), 0.0, 0,
                            stop_lists=stops, budget=budget)
        a, n = int(res["accepted_len"][0]), int(res["emitted_len"][0])
        assert a == K
        E = min(n, a)
        F = int(n == a + 1)
        got = [P + E + F, P + E, P + min(E, K - 1)]
        assert got == case["expect"], case["what"]
        emitted = res["out_tokens"][:n].tolist()
        assert emitted == (drafts + [bonus])[:n]
        assert (res["out_tokens"][n:] == -1).all()


def test_sdcp_example_round_with_stops_and_budgets():
    g = json.load(open(os.path.join(GOLDEN, "sdcp_greedy_round_stops.json")))
    target = _greedy_rows(g["target_argmax"])
    tokens = np.array(g["proposal"], dtype=np.int32)
    cu = offsets_from_depths([len(tokens)])
    for case in g["cases"]:
        budget = [case["budget"]] if case["budget"] is not None else None
        res = oracle.verify(target, None, tokens, cu, 0.0, 0, stop_lists=[case["stop"]], budget=budget, diag=True)
        assert res["accepted_len"][0] == g["expected_accepted"]
        n = int(res["emitted_len"][0])
        assert res["out_tokens"][:n].tolist() == case["emitted"], case
        assert (res["out_tokens"][n:] == -1).all()
        kind = res["terminal_kind"][0]
        assert kind == (oracle.TERM_GREEDY if n == g["expected_accepted"] + 1 else oracle.TERM_NONE)


@pytest.mark.parametrize("temperature", [0.0, 1.0])
def test_truncation_keeps_verdict_and_uniforms(temperature):
    rng = np.random.default_rng(31)
    depths = rng.integers(0, 9, size=200)
    b = make_random("stops", depths, 50, "fp32", temperature, 1.0, 0.5, data_seed=31, verify_seed=5, keep_draft=True)
    base = oracle.verify(b.target, b.draft, b.tokens, b.cu, temperature, 5)
    stops = [list(rng.choice(50, size=rng.integers(0, 4), replace=False)) for _ in range(b.B)]
    budget = rng.integers(-1, 10, size=b.B)
    got = oracle.verify(b.target, b.draft, b.tokens, b.cu, temperature, 5, stop_lists=stops, budget=budget)
    assert np.array_equal(got["accepted_len"], base["accepted_len"])
    for i in range(b.B):
        a = int(base["accepted_len"][i])
        s = slice(b.cu[i] + i, b.cu[i + 1] + i + 1)
        full = base["out_tokens"][s][:a + 1]
        n = int(got["emitted_len"][i])
        assert 0 <= n <= a + 1
        # the emitted tokens are a prefix of the untruncated emission, the rest -1
        assert np.array_equal(got["out_tokens"][s][:n], full[:n])
        assert (got["out_tokens"][s][n:] == -1).all()
        # and the prefix stops exactly where the rule says
        cut = next((j + 1 for j, x in enumerate(full) if x in stops[i]), a + 1)
        assert n == min(cut, max(int(budget[i]), 0))


def test_caller_uniform_zero_is_strict():
    rng = np.random.default_rng(2)
    V, K = 32, 5
    target = rng.standard_normal((K + 1, V)).astype(np.float32)
    draft = (target[:K] + rng.standard_normal((K, V))).astype(np.float32)
    tokens = rng.integers(0, V, size=K).astype(np.int32)
    cu = offsets_from_depths([K])
    r = np.zeros(K)
    u = np.full(K + 1, 0.5)
    res = oracle.verify(target, draft, tokens, cu, 1.0, 0, accept_uniform=r, draw_uniform=u)
    assert res["accepted_len"][0] == K  # r = 0 < p/q whenever p(x) > 0
    target[3, tokens[3]] = -np.inf       # p_3(x_3) = 0: 0 < 0 fails
    res = oracle.verify(target, draft, tokens, cu, 1.0, 0, accept_uniform=r, draw_uniform=u)
    assert res["accepted_len"][0] == 3


def test_caller_uniform_k0_is_searchsorted():
    rng = np.random.default_rng(3)
    B, V = 300, 40
    target = (rng.standard_normal((B, V)) * 2).astype(np.float32)
    u = rng.random(B)
    res = oracle.verify(target, None, np.zeros(0, dtype=np.int32), offsets_from_depths(np.zeros(B, dtype=int)), 0.7,
                        0, accept_uniform=np.zeros(0), draw_uniform=u)
    for i in range(B):
        p = exact.softmax(target[i], 0.7)
        c = np.cumsum(p)
        assert res["out_tokens"][i] == np.searchsorted(c, u[i] * c[-1], side="right")


def test_caller_uniforms_follow_exact_law():
    rng = np.random.default_rng(4)
    K, V, B = 3, 8, 4096
    zt = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
    zd = (zt[:K] + rng.standard_normal((K, V))).astype(np.float32)
    p = np.stack([exact.softmax(r, 1.0) for r in zt])
    q = np.stack([exact.softmax(r, 1.0) for r in zd])
    law = exact.round_distribution(p, q, grid=False)
    cu = offsets_from_depths(np.full(B, K))
    target, draft = np.tile(zt, (B, 1)), np.tile(zd, (B, 1))
    pmf = np.zeros(K + 1)
    reached = np.zeros((K + 1, V))
    for c in range(60):
        g = -np.log(-np.log(np.random.default_rng([6, c]).random((B * K, V))))
        tokens = np.argmax(draft.astype(np.float64) + g, axis=1).astype(np.int32)
        ur = np.random.default_rng([7, c])
        res = oracle.verify(target, draft, tokens, cu, 1.0, 0, accept_uniform=ur.random(B * K),
                            draw_uniform=ur.random(B * (K + 1)))
        a = res["accepted_len"]
        pmf += np.bincount(a, minlength=K + 1)
        slots = res["out_tokens"].reshape(B, K + 1)
        for j in range(K + 1):
            reached[j] += np.bincount(slots[a >= j, j], minlength=V)
    pv = [stats.chisquare(pmf, law["pmf_accepted"] * pmf.sum()).pvalue]
    for j in range(K + 1):
        e = law["token_reached"][j] / law["token_reached"][j].sum() * reached[j].sum()
        pv.append(stats.chisquare(reached[j][e > 0], e[e > 0]).pvalue)
    assert min(pv) * len(pv) > 1e-5, pv


def test_malformed_stop_list_rejects_only_its_request():
    b = make_random("badstops", [2, 3, 1], 20, "fp32", 0.0, 1.0, 0.5, data_seed=1, verify_seed=0)
    offs = np.array([0, 1, 0, 2], dtype=np.int32)  # request 1's list runs backwards
    toks = np.array([5, 6], dtype=np.int32)
    res = oracle.verify(b.target, None, b.tokens, b.cu, 0.0, 0, stop_lists=(offs, toks), diag=True)
    assert res["accepted_len"][1] == -1 and res["emitted_len"][1] == 0
    assert (res["out_tokens"][b.cu[1] + 1: b.cu[2] + 2] == -1).all()
    assert res["accepted_len"][0] >= 0 and res["accepted_len"][2] >= 0
