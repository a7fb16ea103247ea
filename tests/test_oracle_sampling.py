"""Pins for the oracle's Rule 2 (speculative sampling) path.

What fixes the answer, with no implementation to compare against:
  * closed forms of "M7.8 - Speculative Serving", section 0x02 (E[N_commit] = (1-a^(K+1))/(1-a))
    and section 0x02B (P(A=a) = S_a (1 - a_{a+1}), P(A=K) = S_K), also SDCP "Drafting and
    Proposal";
  * losslessness: the emitted tokens follow the target distribution (SDCP Rule 2; "SOTA-227",
    "Why it is free rather than a trade");
  * brute-force enumeration (oracle/exact.py) on tiny vocabularies, checked against both of the
    above, then used as the exact law the oracle's Monte Carlo must reproduce;
  * special cases that reduce to textbook routines (K = 0 is categorical sampling, i.e. numpy's
    searchsorted on the CDF) or are forced (draft == target accepts everything; T -> 0 is greedy);
  * SDCP "Verification and Commit", step 5: q(x) = 0 rejects the request before any draw.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import keying_pins
from oracle import exact, oracle
from workloads import exactness_batch, exactness_case, offsets_from_depths


def _rand_rows(rng, K, V, st=1.5, sd=0.7):
    zt = (rng.standard_normal((K + 1, V)) * st).astype(np.float32)
    zd = (zt[:K] + rng.standard_normal((K, V)) * sd).astype(np.float32)
    return zt, zd


# --------------------------------------------------------------------------- enumeration vs closed forms

@pytest.mark.parametrize("seed", range(6))
def test_enumeration_matches_closed_forms_and_losslessness(seed):
    rng = np.random.default_rng(seed)
    K, V = 3, 8
    zt, zd = _rand_rows(rng, K, V)
    p = np.stack([exact.softmax(r, 1.0) for r in zt])
    q = np.stack([exact.softmax(r, 1.0) for r in zd])
    law = exact.round_distribution(p, q)
    alphas = [exact.acceptance_rate(p[j], q[j]) for j in range(K)]
    S = np.concatenate([[1.0], np.cumprod(alphas)])
    pmf = [S[a] * (1 - alphas[a]) for a in range(K)] + [S[K]]
    np.testing.assert_allclose(law["pmf_accepted"], pmf, rtol=0, atol=1e-13)
    # every emitted position carries exactly the target's distribution
    np.testing.assert_allclose(law["first_token"], p[0], rtol=0, atol=1e-13)
    for j in range(K + 1):
        reach = law["token_reached"][j].sum()
        np.testing.assert_allclose(reach, S[j], rtol=1e-12)
        np.testing.assert_allclose(law["token_reached"][j] / reach, p[j], rtol=0, atol=1e-12)
    mean_c = 1 + S[1:].sum()
    assert np.isclose((np.arange(K + 1) + 1) @ law["pmf_accepted"], mean_c, rtol=1e-13)


def test_enumeration_exact_rationals():
    p = [[Fraction(1, 2), Fraction(1, 3), Fraction(1, 6)],
         [Fraction(1, 5), Fraction(3, 5), Fraction(1, 5)],
         [Fraction(1, 4), Fraction(1, 4), Fraction(1, 2)]]
    q = [[Fraction(1, 3), Fraction(1, 3), Fraction(1, 3)],
         [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)]]
    law = exact.round_distribution_fraction(p, q)
    a0 = sum(min(x, y) for x, y in zip(p[0], q[0]))
    a1 = sum(min(x, y) for x, y in zip(p[1], q[1]))
    assert law["pmf_accepted"] == [1 - a0, a0 * (1 - a1), a0 * a1]
    assert law["token_reached"][0] == p[0]
    assert [x / a0 for x in law["token_reached"][1]] == p[1]
    assert [x / (a0 * a1) for x in law["token_reached"][2]] == p[2]


def test_alpha_point_seven_ledger():
    # the page-2 ledger for alpha = 0.7 (section 0x02A) did not survive extraction; recomputed from
    # E[N_commit] = (1 - a^(K+1)) / (1 - a): 1.7, 2.19, 2.533, 2.7731 for K = 1..4
    p = [Fraction(7, 10), Fraction(3, 10), Fraction(0)]
    q = [Fraction(7, 10), Fraction(0), Fraction(3, 10)]
    expected = [Fraction(17, 10), Fraction(219, 100), Fraction(2533, 1000), Fraction(27731, 10000)]
    for K in range(1, 5):
        law = exact.round_distribution_fraction([p] * (K + 1), [q] * K)
        mean_c = sum((a + 1) * pa for a, pa in enumerate(law["pmf_accepted"]))
        a = Fraction(7, 10)
        assert mean_c == (1 - a ** (K + 1)) / (1 - a) == expected[K - 1]


def test_grid_law_is_within_grid_resolution_of_ideal():
    rng = np.random.default_rng(9)
    zt, zd = _rand_rows(rng, 3, 8)
    p = np.stack([exact.softmax(r, 1.0) for r in zt])
    q = np.stack([exact.softmax(r, 1.0) for r in zd])
    ideal = exact.round_distribution(p, q)
    grid = exact.round_distribution(p, q, grid=True)
    assert np.abs(ideal["pmf_accepted"] - grid["pmf_accepted"]).max() < 8 * 2.0**-24
    assert np.abs(ideal["token_reached"] - grid["token_reached"]).max() < 8 * 2.0**-24


# --------------------------------------------------------------------------- oracle Monte Carlo

def _oracle_monte_carlo(zt, zd, n_calls, B=4096, case_tag=0, rows_differ=False):
    """Histograms of A, y_0 and y_j | reached over n_calls oracle calls of B requests each."""
    K, V = zd.shape[0] if rows_differ else 3, zt.shape[-1]
    pmf = np.zeros(K + 1, dtype=np.int64)
    reached = np.zeros((K + 1, V), dtype=np.int64)
    for c in range(n_calls):
        if rows_differ:
            rng = np.random.Generator(np.random.Philox([77 + case_tag, c]))
            cu = offsets_from_depths(np.full(B, K))
            target = np.ascontiguousarray(np.tile(zt, (B, 1)))
            draft = np.ascontiguousarray(np.tile(zd, (B, 1)))
            g = -np.log(-np.log(rng.random((B * K, V))))
            tokens = np.argmax(draft.astype(np.float64) + g, axis=1).astype(np.int32)
            seed = (case_tag << 40) | c
        else:
            b = exactness_batch(case_tag, c, B=B, rows=(zt, zd))
            target, draft, tokens, cu, seed = b.target, b.draft, b.tokens, b.cu, b.seed
        res = oracle.verify(target, draft, tokens, cu, 1.0, seed)
        a = res["accepted_len"]
        assert (a >= 0).all()
        pmf += np.bincount(a, minlength=K + 1)
        slots = res["out_tokens"].reshape(B, K + 1)
        for j in range(K + 1):
            live = a >= j
            reached[j] += np.bincount(slots[live, j], minlength=V)
    return pmf, reached


def _pvalues(pmf, reached, law):
    n = pmf.sum()
    out = [stats.chisquare(pmf, law["pmf_accepted"] * n).pvalue]
    for j in range(reached.shape[0]):
        m = reached[j].sum()
        e = law["token_reached"][j] / law["token_reached"][j].sum() * m
        keep = e > 0
        assert reached[j][~keep].sum() == 0  # zero-probability tokens are never emitted
        out.append(stats.chisquare(reached[j][keep], e[keep]).pvalue)
    return out


@pytest.mark.parametrize("case,n_calls", [(c, 245) for c in range(8)])
def test_oracle_monte_carlo_matches_exact_law(case, n_calls):
    """Exactness workload: B=4096, K=3, V=8, one fixed row pair per case; 245 calls ~ 10^6 trials."""
    zt, zd = exactness_case(case)
    p = exact.softmax(zt, 1.0)
    q = exact.softmax(zd, 1.0)
    law = exact.round_distribution(np.stack([p] * 4), np.stack([q] * 3), grid=True)
    pmf, reached = _oracle_monte_carlo(zt, zd, n_calls, case_tag=case)
    pv = _pvalues(pmf, reached, law)
    assert min(pv) * len(pv) > 1e-5, pv
    # mean accepted length within 5 sigma of the closed form
    alpha = exact.acceptance_rate(p, q)
    n = pmf.sum()
    mean_a = (np.arange(4) @ pmf) / n
    ea = alpha * (1 - alpha**3) / (1 - alpha)
    var_a = (np.arange(4) ** 2) @ law["pmf_accepted"] - ((np.arange(4)) @ law["pmf_accepted"]) ** 2
    assert abs(mean_a - ea) < 5 * np.sqrt(var_a / n)


def test_oracle_monte_carlo_distinct_rows_per_position():
    """The general, depth-dependent form (section 0x02B) with a different row pair at each position."""
    rng = np.random.default_rng(123)
    zt, zd = _rand_rows(rng, 3, 8, st=1.5, sd=1.0)
    p = np.stack([exact.softmax(r, 1.0) for r in zt])
    q = np.stack([exact.softmax(r, 1.0) for r in zd])
    law = exact.round_distribution(p, q, grid=True)
    pmf, reached = _oracle_monte_carlo(zt, zd, 100, case_tag=99, rows_differ=True)
    pv = _pvalues(pmf, reached, law)
    assert min(pv) * len(pv) > 1e-5, pv


# --------------------------------------------------------------------------- special cases

def test_k0_is_categorical_sampling_by_searchsorted():
    rng = np.random.default_rng(4)
    V, B = 500, 300
    for T in (1.0, 0.7):
        target = (rng.standard_normal((B, V)) * 2.0).astype(np.float32)
        seed = int(rng.integers(1 << 62))
        res = oracle.verify(target, target[:0], np.zeros(0, np.int32), offsets_from_depths(np.zeros(B, int)), T,
                            seed, diag=True)
        assert (res["accepted_len"] == 0).all()
        for i in range(B):
            p = exact.softmax(target[i], T)
            cdf = np.cumsum(p)
            u = (oracle.philox_block(seed, i, 0)[1] >> 8) / 2.0**24
            y = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
            if res["cdf_margin"][i] > 1e-12:
                assert res["out_tokens"][i] == y


def test_bonus_draw_takes_the_block_of_position_k():
    """Every draft accepted (draft rows equal to the target rows): the bonus at t = K_i is the
    categorical draw from p_K with u from Philox block (i, K_i), word 1 (keying_pins)."""
    assert keying_pins.pin_forced_bonus()
    assert keying_pins.pin_forced_bonus(T=0.7, seed=99)


def test_correction_draw_takes_the_block_of_the_rejected_position():
    """A rejection forced at t = 0..3: the correction is the categorical draw from max(p_t - q_t, 0)
    with u from Philox block (i, t), word 1."""
    assert keying_pins.pin_forced_rejection()
    assert keying_pins.pin_forced_rejection(T=1.3, seed=7)


def test_accept_test_takes_word_0_of_the_block_of_its_position():
    """Ratios placed half a 2^-24 step above or below r from block (i, j), word 0, at positions
    j = 0..3: every decision follows that r."""
    assert keying_pins.pin_accept_edges()
    assert keying_pins.pin_accept_edges(seed=2**63 + 12345)


def test_draft_equal_to_target_accepts_everything():
    rng = np.random.default_rng(8)
    depths = rng.integers(0, 10, size=50)
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    V = 64
    target = (rng.standard_normal((n_d + 50, V)) * 3).astype(np.float32)
    t_of_d = np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(50)]).astype(int)
    draft = np.ascontiguousarray(target[t_of_d])
    tokens = rng.integers(0, V, size=n_d).astype(np.int32)
    for seed in range(5):
        res = oracle.verify(target, draft, tokens, cu, 1.0, seed, diag=True)
        assert res["accepted_len"].tolist() == depths.tolist()
        assert (res["ratio"] == 1.0).all()
        assert (res["terminal_kind"] == oracle.TERM_BONUS).all()


def test_single_token_vocabulary():
    depths = [0, 3, 5]
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    target = np.zeros((n_d + 3, 1), dtype=np.float32)
    draft = np.full((n_d, 1), 4.0, dtype=np.float32)
    res = oracle.verify(target, draft, np.zeros(n_d, np.int32), cu, 1.0, 5)
    assert res["accepted_len"].tolist() == depths
    assert (res["out_tokens"] == 0).all()


def test_low_temperature_sampling_converges_to_greedy():
    rng = np.random.default_rng(10)
    depths = rng.integers(0, 6, size=30)
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    V = 40
    target = (rng.standard_normal((n_d + 30, V)) * 2).astype(np.float32)
    top = np.argmax(target, axis=1)
    target[np.arange(target.shape[0]), top] += 1.0  # a clear winner on every row
    t_of_d = np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(30)]).astype(int)
    draft = (target[t_of_d] + rng.standard_normal((n_d, V)) * 1.5).astype(np.float32)
    dtop = np.argmax(draft, axis=1)
    draft[np.arange(n_d), dtop] += 1.0
    tokens = np.argmax(draft, axis=1).astype(np.int32)
    greedy = oracle.verify(target, None, tokens, cu, 0.0, 0)
    cold = oracle.verify(target, draft, tokens, cu, 1e-3, 123)
    assert cold["accepted_len"].tolist() == greedy["accepted_len"].tolist()
    assert cold["out_tokens"].tolist() == greedy["out_tokens"].tolist()


# --------------------------------------------------------------------------- preconditions and invariants

def test_zero_draft_probability_rejects_before_any_draw():
    rng = np.random.default_rng(12)
    depths = [3, 2, 0, 4]
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    V = 20
    target = rng.standard_normal((n_d + 4, V)).astype(np.float32)
    draft = rng.standard_normal((n_d, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=n_d).astype(np.int32)
    base = oracle.verify(target, draft, tokens, cu, 1.0, 77)
    bad = draft.copy()
    bad[cu[1] + 1, tokens[cu[1] + 1]] = -np.inf  # request 1, position 1: q(x) = 0
    res = oracle.verify(target, bad, tokens, cu, 1.0, 77)
    assert res["accepted_len"].tolist() == [base["accepted_len"][0], -1, base["accepted_len"][2], base["accepted_len"][3]]
    assert (res["out_tokens"][cu[1] + 1: cu[2] + 2] == -1).all()
    others = np.ones(n_d + 4, bool)
    others[cu[1] + 1: cu[2] + 2] = False
    assert (res["out_tokens"][others] == base["out_tokens"][others]).all()


def test_depth_limit_and_token_range():
    rng = np.random.default_rng(13)
    depths = [65, 2]
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    V = 10
    target = rng.standard_normal((n_d + 2, V)).astype(np.float32)
    draft = rng.standard_normal((n_d, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=n_d).astype(np.int32)
    res = oracle.verify(target, draft, tokens, cu, 1.0, 1)
    assert res["accepted_len"][0] == -1 and res["accepted_len"][1] >= 0
    tokens[-1] = -3
    res = oracle.verify(target, draft, tokens, cu, 1.0, 1)
    assert res["accepted_len"][1] == -1 and (res["out_tokens"][cu[1] + 1:] == -1).all()


def test_ragged_batch_invariants():
    rng = np.random.default_rng(14)
    B, V = 64, 300
    depths = rng.integers(0, 13, size=B)
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    target = (rng.standard_normal((n_d + B, V)) * 2).astype(np.float32)
    t_of_d = np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(B)]).astype(int)
    draft = (target[t_of_d] + rng.standard_normal((n_d, V)) * 1.0).astype(np.float32)
    g = -np.log(-np.log(rng.random((n_d, V))))
    tokens = np.argmax(draft.astype(np.float64) + g, axis=1).astype(np.int32)
    for seed in range(4):
        res = oracle.verify(target, draft, tokens, cu, 1.0, seed, diag=True)
        for i in range(B):
            K, a, base = int(depths[i]), int(res["accepted_len"][i]), int(cu[i] + i)
            assert 0 <= a <= K  # at least one and at most K + 1 tokens per round
            slots = res["out_tokens"][base: base + K + 1]
            assert slots[:a].tolist() == tokens[cu[i]: cu[i] + a].tolist()
            assert (slots[a + 1:] == -1).all() and 0 <= slots[a] < V
            y = slots[a]
            pt = exact.softmax(target[base + a], 1.0)
            if a < K:
                assert res["terminal_kind"][i] == oracle.TERM_RESIDUAL
                qt = exact.softmax(draft[cu[i] + a], 1.0)
                assert pt[y] > qt[y]  # the correction comes from the positive part of p - q
            else:
                assert res["terminal_kind"][i] == oracle.TERM_BONUS and pt[y] > 0
