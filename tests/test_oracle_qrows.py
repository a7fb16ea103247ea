"""Pins for the oracle's probability-row draft input (SDCP's "q_rows": each proposed position
carries the draft distribution itself as V binary32 values; section "Message Definitions", and
Rule 2 of section "Acceptance Rules", which uses q[i] from those rows).

What fixes the answer:
  * with q rows equal to the draft softmax rounded to binary32, the verdicts equal those of the
    logit path up to decisions within 1e-6 of their thresholds (the rounding moves p/q by ~1e-7);
  * Monte Carlo against the exact law of the method (enumeration) with the given q rows;
  * a proposal whose q at its token is zero is rejected before any draw (SDCP "Verification and
    Commit", step 5); Rule 1 never reads q.
"""
import numpy as np
import pytest
from scipy import stats

from oracle import exact, oracle
from oracle.compare import compare_verdicts
from workloads import make_random, offsets_from_depths


def _softmax_rows(z, T):
    z = z.astype(np.float64) / T
    z -= z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("T,dtype", [(1.0, "fp32"), (0.7, "bf16")])
def test_qrows_equal_to_draft_softmax_match_the_logit_path(T, dtype):
    rng = np.random.default_rng(4)
    b = make_random("qrows", rng.integers(0, 9, size=150), 300, dtype, T, 2.0, 1.0, data_seed=4, verify_seed=9)
    q = _softmax_rows(b.draft_f32(), T).astype(np.float32)
    ref = oracle.verify(b.target, b.draft, b.tokens, b.cu, T, 9, diag=True)
    got = oracle.verify(b.target, None, b.tokens, b.cu, T, 9, draft_probs=q, diag=True)
    cmp = compare_verdicts(got["accepted_len"], got["out_tokens"], ref, b.cu, T)
    assert cmp["n_hard"] == 0, cmp["hard"][:5]
    np.testing.assert_allclose(got["ratio"], ref["ratio"], rtol=1e-6)
    assert np.isnan(got["draft_lse"]).all()  # no draft log-normaliser exists for given rows


def test_qrows_monte_carlo_follows_exact_law():
    rng = np.random.default_rng(8)
    K, V, B = 3, 8, 4096
    zt = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
    qd = rng.dirichlet(np.full(V, 0.8), size=K)
    qd[:, 0] = 0.0  # a token the drafter never proposes: q = 0 there, p > 0
    q32 = (qd / qd.sum(axis=1, keepdims=True)).astype(np.float32)  # a distribution, rounded to binary32
    q = q32.astype(np.float64) / q32.astype(np.float64).sum(axis=1, keepdims=True)
    p = np.stack([exact.softmax(r, 1.0) for r in zt])
    law = exact.round_distribution(p, q, grid=True)
    cu = offsets_from_depths(np.full(B, K))
    target = np.tile(zt, (B, 1))
    qrows = np.tile(q32, (B, 1))
    pmf = np.zeros(K + 1)
    reached = np.zeros((K + 1, V))
    with np.errstate(divide="ignore"):
        logq = np.log(np.tile(q, (B, 1)))
    for c in range(60):
        g = -np.log(-np.log(np.random.default_rng([10, c]).random((B * K, V))))
        tokens = np.argmax(logq + g, axis=1).astype(np.int32)
        res = oracle.verify(target, None, tokens, cu, 1.0, 500 + c, draft_probs=qrows)
        a = res["accepted_len"]
        assert (a >= 0).all()
        pmf += np.bincount(a, minlength=K + 1)
        slots = res["out_tokens"].reshape(B, K + 1)
        for j in range(K + 1):
            reached[j] += np.bincount(slots[a >= j, j], minlength=V)
    pv = [stats.chisquare(pmf, law["pmf_accepted"] * pmf.sum()).pvalue]
    for j in range(K + 1):
        e = law["token_reached"][j] / law["token_reached"][j].sum() * reached[j].sum()
        assert reached[j][e == 0].sum() == 0
        pv.append(stats.chisquare(reached[j][e > 0], e[e > 0]).pvalue)
    assert min(pv) * len(pv) > 1e-5, pv


def test_zero_q_at_the_token_rejects_before_any_draw():
    rng = np.random.default_rng(5)
    b = make_random("qzero", [3, 2, 4], 50, "fp32", 1.0, 2.0, 1.0, data_seed=5, verify_seed=1)
    q = _softmax_rows(b.draft_f32(), 1.0).astype(np.float32)
    d = b.cu[1] + 1  # second draft row of request 1
    q[d, b.tokens[d]] = 0.0
    got = oracle.verify(b.target, None, b.tokens, b.cu, 1.0, 1, draft_probs=q, diag=True)
    assert got["accepted_len"][1] == -1 and got["terminal_kind"][1] == oracle.TERM_BAD
    assert (got["out_tokens"][b.cu[1] + 1: b.cu[2] + 2] == -1).all()
    assert got["accepted_len"][0] >= 0 and got["accepted_len"][2] >= 0


def test_greedy_never_reads_q():
    b = make_random("qgreedy", [3, 0, 5], 40, "fp32", 0.0, 2.0, 1.0, data_seed=6, verify_seed=0, keep_draft=True)
    q = np.full((b.n_draft_rows, b.V), np.nan, dtype=np.float32)
    got = oracle.verify(b.target, None, b.tokens, b.cu, 0.0, 0, draft_probs=q)
    ref = oracle.verify(b.target, None, b.tokens, b.cu, 0.0, 0)
    assert np.array_equal(got["accepted_len"], ref["accepted_len"])
    assert np.array_equal(got["out_tokens"], ref["out_tokens"])
