"""Pins for the oracle's per-request sampling profiles (temperature and seed per request).

SDCP "Session Contract" gives every session its own sampling profile; a verification batch gathers
requests of many sessions.  What fixes the answer:
  * request i of a profiled batch must verify exactly as request i of the same batch verified with
    the scalar profile (T_i, seed_i) - the scalar path is pinned by enumeration, closed forms and
    Monte Carlo elsewhere;
  * a batch mixing two temperatures must follow, group by group, the exact law of the method at
    each group's temperature (brute-force enumeration, oracle/exact.py);
  * a temperature that describes no profile (negative, NaN, infinite) rejects that request alone.
"""
import numpy as np
import pytest
from scipy import stats

from oracle import exact, oracle
from workloads import make_random, offsets_from_depths

PROFILES = [(0.0, 11), (0.7, 12), (1.0, 13), (1.6, 0xFFFFFFFF00000001)]


def _ragged(V=257, B=24, dtype="fp32", seed=5):
    rng = np.random.default_rng(seed)
    depths = rng.integers(0, 7, size=B)
    return make_random("profiles", depths, V, dtype, 1.0, 2.0, 1.0, data_seed=seed, verify_seed=0)


def _slots(res, cu, i):
    return res["out_tokens"][cu[i] + i: cu[i + 1] + i + 1]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_profiled_request_equals_scalar_run_with_its_profile(dtype):
    b = _ragged(dtype=dtype)
    rng = np.random.default_rng(1)
    pick = rng.integers(0, len(PROFILES), size=b.B)
    T = np.array([PROFILES[k][0] for k in pick])
    seeds = np.array([PROFILES[k][1] for k in pick], dtype=np.uint64)
    got = oracle.verify(b.target, b.draft, b.tokens, b.cu, T, seeds)
    scalar = {k: oracle.verify(b.target, b.draft, b.tokens, b.cu, PROFILES[k][0], PROFILES[k][1])
              for k in range(len(PROFILES))}
    for i in range(b.B):
        ref = scalar[pick[i]]
        assert got["accepted_len"][i] == ref["accepted_len"][i], i
        assert np.array_equal(_slots(got, b.cu, i), _slots(ref, b.cu, i)), i
    assert len(set(pick)) == len(PROFILES)


@pytest.mark.parametrize("bad_T", [-1.0, float("nan"), float("inf"), -0.0 - 1e-30])
def test_invalid_temperature_rejects_only_its_request(bad_T):
    b = _ragged()
    T = np.full(b.B, 1.0)
    T[5] = bad_T
    seeds = np.full(b.B, 77, dtype=np.uint64)
    got = oracle.verify(b.target, b.draft, b.tokens, b.cu, T, seeds, diag=True)
    ref = oracle.verify(b.target, b.draft, b.tokens, b.cu, 1.0, 77)
    assert got["accepted_len"][5] == -1
    assert (_slots(got, b.cu, 5) == -1).all()
    assert got["terminal_kind"][5] == oracle.TERM_BAD
    keep = np.arange(b.B) != 5
    assert np.array_equal(got["accepted_len"][keep], ref["accepted_len"][keep])
    for i in np.nonzero(keep)[0]:
        assert np.array_equal(_slots(got, b.cu, i), _slots(ref, b.cu, i))


def test_mixed_temperatures_follow_each_groups_exact_law():
    """B = 4096 requests of depth 3 over V = 8, distinct rows per position; even requests at T = 0.7,
    odd ones at T = 1.4; 60 calls.  Each group's histograms against the exact law at its T."""
    rng = np.random.default_rng(2024)
    K, V, B = 3, 8, 4096
    zt = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
    zd = (zt[:K] + rng.standard_normal((K, V)) * 1.0).astype(np.float32)
    temps = (0.7, 1.4)
    laws = []
    for T in temps:
        p = np.stack([exact.softmax(r, T) for r in zt])
        q = np.stack([exact.softmax(r, T) for r in zd])
        laws.append(exact.round_distribution(p, q, grid=True))
    cu = offsets_from_depths(np.full(B, K))
    target, draft = np.tile(zt, (B, 1)), np.tile(zd, (B, 1))
    T_each = np.where(np.arange(B) % 2 == 0, temps[0], temps[1])
    pmf = np.zeros((2, K + 1))
    reached = np.zeros((2, K + 1, V))
    for c in range(60):
        g = -np.log(-np.log(np.random.default_rng([9, c]).random((B * K, V))))
        t_rows = np.repeat(T_each, K)[:, None]
        tokens = np.argmax(draft.astype(np.float64) / t_rows + g, axis=1).astype(np.int32)
        seeds = np.arange(B, dtype=np.uint64) * np.uint64(1000003) + np.uint64(c)
        res = oracle.verify(target, draft, tokens, cu, T_each, seeds)
        a = res["accepted_len"]
        assert (a >= 0).all()
        slots = res["out_tokens"].reshape(B, K + 1)
        for grp in range(2):
            sel = np.arange(B) % 2 == grp
            pmf[grp] += np.bincount(a[sel], minlength=K + 1)
            for j in range(K + 1):
                reached[grp, j] += np.bincount(slots[sel & (a >= j), j], minlength=V)
    pv = []
    for grp in range(2):
        law = laws[grp]
        pv.append(stats.chisquare(pmf[grp], law["pmf_accepted"] * pmf[grp].sum()).pvalue)
        for j in range(K + 1):
            e = law["token_reached"][j] / law["token_reached"][j].sum() * reached[grp, j].sum()
            assert reached[grp, j][e == 0].sum() == 0
            pv.append(stats.chisquare(reached[grp, j][e > 0], e[e > 0]).pvalue)
    assert min(pv) * len(pv) > 1e-5, pv
    # the two groups really differ: their exact accepted-length laws are far apart
    assert np.abs(laws[0]["pmf_accepted"] - laws[1]["pmf_accepted"]).max() > 0.02
