"""Pins of the oracle's top-k / top-p truncation, each usable against a mutated oracle build.

TEST INFRASTRUCTURE ONLY.  SDCP ("Speculative Decoding Coordination Protocol (SDCP)", section
"Session Contract") defines p as the model's distribution after temperature, then top-k, then
top-p.  The oracle sorts each row into rank order and cuts it.  The pins here do not sort:

  * hand-worked cases (tests/golden/top_k_top_p.json);
  * the per-token form of the same definition on tiny rows full of ties: token v is kept iff
    fewer than top_k tokens rank before it, and (when top-p applies) it ranks first or the mass of
    the top-k tokens ranked before it is still short of the nucleus mass.  Counting the tokens and
    summing the mass that rank before each token is a different computation from sorting, and the
    two agree exactly when the definition is implemented right;
  * top_k = 1 at any temperature reduces Rule 2 to Rule 1 (the greedy rule): p and q become point
    masses on the two argmaxes, smallest id on ties;
  * the exact law of a round with truncated rows (oracle/exact.py enumerates it from the
    truncated distributions built here) against a Monte Carlo of the oracle;
  * a profile that truncates nothing leaves every verdict unchanged, and one that describes no
    profile rejects its request alone.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy import stats

from oracle import exact, oracle
from workloads import offsets_from_depths

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "top_k_top_p.json")


def kept_by_definition(z, T: float, top_k: int, top_p_milli: int) -> np.ndarray:
    """The kept tokens of one row, token by token, without sorting (see the module docstring)."""
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    ids = np.arange(V)
    e = np.exp((z - z.max()) / T)
    # ahead[u, v]: token u ranks before token v (larger logit, or equal logit and smaller id)
    ahead = (z[:, None] > z[None, :]) | ((z[:, None] == z[None, :]) & (ids[:, None] < ids[None, :]))
    n_ahead = ahead.sum(axis=0)
    in_k = n_ahead < top_k if 0 < top_k < V else np.ones(V, dtype=bool)
    if top_p_milli >= 1000:
        return in_k
    mass_k = e[in_k].sum()
    mass_ahead = (ahead * (e * in_k)[:, None]).sum(axis=0)
    return in_k & ((n_ahead == 0) | (mass_ahead < mass_k * (top_p_milli / 1000.0)))


def truncated_softmax(z, T: float, top_k: int, top_p_milli: int) -> np.ndarray:
    p = exact.softmax(z, T) * kept_by_definition(z, T, top_k, top_p_milli)
    return p / p.sum()


def pin_worked_examples(lib_path: str = oracle.LIBRARY) -> bool:
    for case in json.load(open(GOLDEN))["cases"]:
        with np.errstate(divide="ignore"):
            z = np.log(np.asarray(case["weights"], dtype=np.float64)).astype(np.float32)
        got = oracle.truncate_row(z, case["T"], case["top_k"], case["top_p_milli"], lib_path=lib_path)
        if np.nonzero(got["keep"])[0].tolist() != case["kept"] or got["n"] != len(case["kept"]):
            return False
    return True


def pin_definition(lib_path: str = oracle.LIBRARY, n_rows: int = 400) -> bool:
    """Random tiny rows drawn from a few distinct values (so ties are everywhere), bf16 and fp32,
    against the per-token definition.  Rows whose top-p decision sits within 1e-9 of its
    threshold are skipped: there the two summation orders may round to different sides."""
    rng = np.random.default_rng(2024)
    for n in range(n_rows):
        V = int(rng.integers(1, 14))
        levels = rng.standard_normal(int(rng.integers(1, 5))) * 2.0
        z = rng.choice(levels, size=V).astype(np.float32)
        if rng.random() < 0.2:
            z[rng.integers(0, V)] = -np.inf
        if not np.isfinite(z).any():
            z[0] = 0.0
        T = float(rng.choice([0.5, 1.0, 1.7]))
        top_k = int(rng.choice([0, 1, 2, 3, V - 1, V, V + 3]))
        milli = int(rng.choice([0, 1, 250, 500, 800, 950, 999, 1000]))
        # even rows as bf16: the top half of the binary32 bits; the definition reads the stored values
        row = z if n % 2 else (z.view(np.uint32) >> 16).astype(np.uint16)
        zz = z if n % 2 else (row.astype(np.uint32) << 16).view(np.float32)
        got = oracle.truncate_row(row, T, top_k, milli, lib_path=lib_path)
        if got["margin"] < 1e-9:
            continue
        want = kept_by_definition(zz, T, top_k, milli)
        if not np.array_equal(got["keep"], want) or got["n"] != int(want.sum()):
            return False
        lse = zz.astype(np.float64).max() / T + np.log(np.exp((zz[want].astype(np.float64) - zz.max()) / T).sum())
        if abs(got["lse_kept"] - lse) > 1e-12 * max(1.0, abs(lse)):
            return False
    return True


def pin_greedy_reduction(lib_path: str = oracle.LIBRARY) -> bool:
    """top_k = 1 at T > 0 gives Rule 1's verdicts when every draft is its row's argmax."""
    rng = np.random.default_rng(77)
    depths = rng.integers(0, 6, size=40)
    cu = offsets_from_depths(depths)
    n_d, B, V = int(cu[-1]), 40, 50
    # few distinct values: ties at the maximum are common in both target and draft rows
    target = rng.integers(-3, 4, size=(n_d + B, V)).astype(np.float32)
    draft = rng.integers(-3, 4, size=(n_d, V)).astype(np.float32)
    tokens = np.argmax(draft, axis=1).astype(np.int32)  # the first maximum: the smallest id
    # half the requests draft the target argmax, so acceptances happen
    for i in range(0, B, 2):
        for j in range(int(depths[i])):
            r = cu[i] + i + j
            draft[cu[i] + j] = target[r]
            tokens[cu[i] + j] = int(np.argmax(target[r]))
    greedy = oracle.verify(target, None, tokens, cu, 0.0, 0, lib_path=lib_path)
    for T in (0.3, 1.0, 2.5):
        got = oracle.verify(target, draft, tokens, cu, T, 5, lib_path=lib_path, top_k=np.ones(B, dtype=np.int32))
        if not (np.array_equal(got["accepted_len"], greedy["accepted_len"])
                and np.array_equal(got["out_tokens"], greedy["out_tokens"])):
            return False
        if (got["kept_tokens"][: n_d + B] != 1).any() or (got["kept_tokens"][n_d + B:] != 1).any():
            return False
    return True


def pin_no_truncation_and_invalid(lib_path: str = oracle.LIBRARY) -> bool:
    rng = np.random.default_rng(31)
    depths = rng.integers(0, 5, size=16)
    cu = offsets_from_depths(depths)
    n_d, B, V = int(cu[-1]), 16, 40
    target = (rng.standard_normal((n_d + B, V)) * 2).astype(np.float32)
    draft = (target[:n_d] + rng.standard_normal((n_d, V))).astype(np.float32)
    tokens = rng.integers(0, V, size=n_d).astype(np.int32)
    ref = oracle.verify(target, draft, tokens, cu, 0.9, 4, lib_path=lib_path, diag=True)
    top_k = rng.choice([0, V, V + 5], size=B).astype(np.int32)
    got = oracle.verify(target, draft, tokens, cu, 0.9, 4, lib_path=lib_path, diag=True, top_k=top_k,
                        top_p_milli=np.full(B, 1000, dtype=np.int32))
    if not (np.array_equal(got["accepted_len"], ref["accepted_len"])
            and np.array_equal(got["out_tokens"], ref["out_tokens"])
            and np.array_equal(got["target_lse"], ref["target_lse"])):
        return False
    valid = ref["accepted_len"] >= 0
    rows_t = np.concatenate([np.arange(cu[i] + i, cu[i + 1] + i + 1) for i in np.nonzero(valid)[0]])
    if (got["kept_tokens"][rows_t] != V).any():
        return False
    bad_k, bad_p = top_k.copy(), np.full(B, 1000, dtype=np.int32)
    bad_k[3], bad_p[5], bad_p[6] = -1, 1001, -2
    got = oracle.verify(target, draft, tokens, cu, 0.9, 4, lib_path=lib_path, top_k=bad_k, top_p_milli=bad_p)
    others = np.setdiff1d(np.arange(B), [3, 5, 6])
    if not (got["accepted_len"][[3, 5, 6]] == -1).all():
        return False
    if not np.array_equal(got["accepted_len"][others], ref["accepted_len"][others]):
        return False
    # a greedy request with an invalid profile is rejected too; a valid one ignores the profile
    g = oracle.verify(target, None, tokens, cu, 0.0, 0, lib_path=lib_path, top_k=bad_k, top_p_milli=bad_p)
    g0 = oracle.verify(target, None, tokens, cu, 0.0, 0, lib_path=lib_path)
    return (g["accepted_len"][[3, 5, 6]] == -1).all() and np.array_equal(g["accepted_len"][others],
                                                                          g0["accepted_len"][others])


def pin_monte_carlo(lib_path: str = oracle.LIBRARY, calls: int = 40) -> bool:
    """K = 3, V = 8, one truncating profile per case; drafts drawn from the truncated q.  The
    accepted-length law and the token law at every position must match the exact enumeration
    over the truncated rows built by the per-token definition (chi-square p > 1e-6)."""
    rng = np.random.default_rng(909)
    K, V, B, T = 3, 8, 4096, 0.8
    ok = True
    for top_k, milli in ((5, 1000), (0, 900), (6, 850)):
        zt = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
        zd = (zt[:K] + rng.standard_normal((K, V)) * 1.0).astype(np.float32)
        p = np.stack([truncated_softmax(r, T, top_k, milli) for r in zt])
        q = np.stack([truncated_softmax(r, T, top_k, milli) for r in zd])
        law = exact.round_distribution(p, q, grid=True)
        cu = offsets_from_depths(np.full(B, K))
        target, draft = np.tile(zt, (B, 1)), np.tile(zd, (B, 1))
        with np.errstate(divide="ignore"):
            logq = np.log(np.tile(q, (B, 1)))
        pmf = np.zeros(K + 1)
        reached = np.zeros((K + 1, V))
        for c in range(calls):
            g = -np.log(-np.log(np.random.default_rng([11, top_k, milli, c]).random((B * K, V))))
            with np.errstate(invalid="ignore"):
                tokens = np.argmax(logq + g, axis=1).astype(np.int32)
            res = oracle.verify(target, draft, tokens, cu, T, 7000 + c, lib_path=lib_path,
                                top_k=np.full(B, top_k, dtype=np.int32), top_p_milli=np.full(B, milli, dtype=np.int32))
            a = res["accepted_len"]
            if (a < 0).any():
                return False
            pmf += np.bincount(a, minlength=K + 1)
            slots = res["out_tokens"].reshape(B, K + 1)
            for j in range(K + 1):
                reached[j] += np.bincount(np.clip(slots[a >= j, j], 0, V - 1), minlength=V)
        pv = []
        # cells the exact law gives probability 0 must stay empty; the others are tested together
        for obs, prob in [(pmf, law["pmf_accepted"])] + [(reached[j], law["token_reached"][j]) for j in range(K + 1)]:
            e = prob / prob.sum() * obs.sum()
            if (obs[e == 0] > 0).any():
                return False
            if (e > 0).sum() > 1:
                pv.append(stats.chisquare(obs[e > 0], e[e > 0]).pvalue)
        ok &= min(pv) > 1e-6
    return ok


ALL = (pin_worked_examples, pin_definition, pin_greedy_reduction, pin_no_truncation_and_invalid, pin_monte_carlo)
