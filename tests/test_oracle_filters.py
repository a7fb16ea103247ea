"""The oracle's top-k / top-p truncation against its pins (SDCP "Session Contract": temperature,
then top-k, then top-p).  The pins themselves are in filter_pins.py, shared with the mutation test.
"""
import numpy as np

import filter_pins as F
from oracle import exact, oracle
from workloads import offsets_from_depths


def test_hand_worked_cases():
    assert F.pin_worked_examples()


def test_sorting_cut_equals_per_token_definition():
    assert F.pin_definition(n_rows=2000)


def test_top_k_one_is_the_greedy_rule():
    assert F.pin_greedy_reduction()


def test_profiles_that_truncate_nothing_and_invalid_profiles():
    assert F.pin_no_truncation_and_invalid()


def test_truncated_round_has_the_exact_law():
    assert F.pin_monte_carlo(calls=60)


def test_lossless_under_truncation_exact_enumeration():
    """With truncated p and q the emitted token at every reached position has law p' exactly
    (SOTA-227, "Why it is free rather than a trade"; SDCP Rule 2), whatever the truncation does to
    q: the enumeration over all draft tuples shows it to 1e-12."""
    rng = np.random.default_rng(3)
    K, V, T = 3, 7, 1.1
    for top_k, milli in ((3, 1000), (0, 600), (5, 900), (2, 0)):
        zt = rng.standard_normal((K + 1, V)) * 1.5
        zd = zt[:K] + rng.standard_normal((K, V))
        p = np.stack([F.truncated_softmax(r, T, top_k, milli) for r in zt])
        q = np.stack([F.truncated_softmax(r, T, top_k, milli) for r in zd])
        law = exact.round_distribution(p, q)
        for j in range(K + 1):
            reached = law["token_reached"][j]
            if reached.sum() > 0:  # point masses on different tokens reject at position 0 every time
                np.testing.assert_allclose(reached / reached.sum(), p[j], atol=1e-12)
        assert law["token_reached"][0].sum() > 0


def test_kept_counts_lses_and_margins_in_the_batch_layout():
    rng = np.random.default_rng(19)
    depths = rng.integers(0, 5, size=24)
    cu = offsets_from_depths(depths)
    n_d, B, V = int(cu[-1]), 24, 300
    target = (rng.standard_normal((n_d + B, V)) * 2).astype(np.float32)
    draft = (target[:n_d] + rng.standard_normal((n_d, V)) * 0.5).astype(np.float32)
    top_k = rng.choice([0, 1, 20, 100], size=B).astype(np.int32)
    milli = rng.choice([1000, 900, 500], size=B).astype(np.int32)
    # drafts drawn from the truncated draft rows so that no request is a bad proposal
    tokens = np.zeros(n_d, dtype=np.int32)
    for i in range(B):
        for j in range(int(depths[i])):
            q = F.truncated_softmax(draft[cu[i] + j], 0.7, int(top_k[i]), int(milli[i]))
            tokens[cu[i] + j] = rng.choice(V, p=q)
    res = oracle.verify(target, draft, tokens, cu, 0.7, 9, diag=True, top_k=top_k, top_p_milli=milli)
    assert (res["accepted_len"] >= 0).all()
    n_t = n_d + B
    for i in range(B):
        rows = [(cu[i] + i + j, target[cu[i] + i + j]) for j in range(int(depths[i]) + 1)]
        rows += [(n_t + cu[i] + j, draft[cu[i] + j]) for j in range(int(depths[i]))]
        for slot, z in rows:
            keep = F.kept_by_definition(z, 0.7, int(top_k[i]), int(milli[i]))
            assert res["kept_tokens"][slot] == keep.sum()
            if milli[i] == 1000:
                assert res["filter_margin"][slot] == np.inf
            else:
                assert 0.0 <= res["filter_margin"][slot] < 1.0
        for j in range(int(depths[i]) + 1):
            r = cu[i] + i + j
            keep = F.kept_by_definition(target[r], 0.7, int(top_k[i]), int(milli[i]))
            z = target[r].astype(np.float64) / 0.7
            want = z.max() + np.log(np.exp(z[keep] - z.max()).sum())
            assert abs(res["target_lse"][r] - want) < 1e-12 * abs(want) + 1e-12


def test_given_probability_rows_truncate_only_p():
    """With SDCP q_rows the drafter's distribution is taken as given; the profile truncates p."""
    rng = np.random.default_rng(23)
    B, K, V, T = 400, 3, 10, 1.0
    cu = offsets_from_depths(np.full(B, K))
    zt = rng.standard_normal((K + 1, V)).astype(np.float32) * 2
    q_row = rng.dirichlet(np.ones(V), size=K).astype(np.float32)
    q_row /= q_row.sum(axis=1, keepdims=True)
    target = np.tile(zt, (B, 1))
    probs = np.tile(q_row, (B, 1))
    tokens = np.array([rng.choice(V, p=probs[d] / probs[d].sum()) for d in range(B * K)], dtype=np.int32)
    res = oracle.verify(target, None, tokens, cu, T, 2, diag=True, draft_probs=probs,
                        top_k=np.full(B, 4, dtype=np.int32))
    assert (res["accepted_len"] >= 0).all()
    keep = np.stack([F.kept_by_definition(r, T, 4, 1000) for r in zt])
    p = np.stack([F.truncated_softmax(r, T, 4, 1000) for r in zt])
    for i in range(B):
        for j in range(K):
            d = i * K + j
            x = tokens[d]
            want = p[j][x] / probs[d][x]
            assert abs(res["ratio"][d] - want) <= 1e-12 * max(want, 1.0)
    # every emitted token is one the truncated target keeps
    slots = res["out_tokens"].reshape(B, K + 1)
    a = res["accepted_len"]
    for i in range(B):
        y = slots[i, a[i]]
        assert keep[a[i]][y]
    assert (res["kept_tokens"][: B * K + B] == 4).all()
