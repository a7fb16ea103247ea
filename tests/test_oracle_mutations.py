"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU only), builds it, and
checks that at least one pin fails: the Monte Carlo against the exact enumeration, the
closed-form LSE, the planted argmax tie, the rocRAND Philox values, the per-request profile
check (each request of a profiled batch against the scalar run with its own profile), or the
top-k / top-p pins of filter_pins.py.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

import filter_pins
import keying_pins
import tree_pins
from oracle import exact, oracle
from workloads import offsets_from_depths

HERE = os.path.dirname(os.path.abspath(__file__))

MUTATIONS = {
    "residual_without_clamp": ("w[v] = p > q ? p - q : 0.0;", "w[v] = p - q;"),
    "residual_sign_flipped": ("w[v] = p > q ? p - q : 0.0;", "w[v] = q > p ? q - p : 0.0;"),
    "ratio_inverted": ("ratio = exp(log_ratio);", "ratio = exp(-log_ratio);"),
    "accept_comparison_reversed": ("accept = r <= ratio;", "accept = r >= ratio;"),
    "caller_accept_not_strict": ("accept = r < ratio;", "accept = r <= ratio;"),
    "stop_token_not_emitted": ("n = j + 1;\n      break;", "n = j;\n      break;"),
    "budget_ignored": ("if (b < n) n = b;", "(void)b;"),
    "frontier_drawn_after_stop": ("if (n_emit < a + 1) {", "if (n_emit < a) {"),
    "caller_draw_uniform_of_first_position": ("u = opt->draw_uniform[trow0 + t];", "u = opt->draw_uniform[trow0];"),
    "lse_drops_max": ("return m / T + log(s);", "return log(s);"),
    "residual_from_next_row": ("const double p = kept(keep_t, t, V, v) ? exp(logit_at(target, dtype, trow0 + t, V, v) / T - lse_t[t]) : 0.0;",
                               "const double p = exp(logit_at(target, dtype, trow0 + t + 1, V, v) / T - lse_t[t + 1]);"),
    "bonus_from_draft_side": ("      w[v] = kept(keep_t, t, V, v) ? exp(logit_at(target, dtype, trow0 + t, V, v) / T - lse_t[t]) : 0.0;\n  }\n  double S, margin;",
                              "      w[v] = exp(logit_at(target, dtype, trow0 + t, V, v) / T - lse_t[t]) * (v + 1);\n  }\n  double S, margin;"),
    "greedy_tie_to_largest": ("if (z > best_z) {", "if (z >= best_z) {"),
    "philox_key_bumped_every_round": ("if (round > 0) {", "if (round >= 0) {"),
    "profile_temperature_of_first_request": ("T_each ? T_each[i] : T", "T_each ? T_each[0] : T"),
    "profile_seed_of_next_request": ("seed_each ? seed_each[i] : seed", "seed_each ? seed_each[(i + 1) % B] : seed"),
    "profile_invalid_temperature_accepted": ("int bad = !(T >= 0.0) || isinf(T) ||", "int bad = 0 ||"),
    "qrows_ratio_not_divided": ("lse_t[j]) / (double)qrows[(drow0 + j) * (int64_t)V + x];", "lse_t[j]);"),
    "qrows_residual_from_wrong_row": ("const double q = qrows ? (double)qrows[(drow0 + t) * (int64_t)V + v]",
                                      "const double q = qrows ? (double)qrows[(drow0 + (t > 0 ? t - 1 : t + 1)) * (int64_t)V + v]"),
    "temperature_ignored": ("drow0 + j, V, x)) / T - (lse_t[j] - lse_d[j]);", "drow0 + j, V, x)) - (lse_t[j] - lse_d[j]);"),
    # top-k / top-p
    "rank_ties_to_larger_id": ("return a->v < b->v ? -1 : (a->v > b->v);", "return a->v > b->v ? -1 : (a->v < b->v);"),
    "top_k_off_by_one": ("int64_t n = (top_k > 0 && top_k < V) ? top_k : V;",
                         "int64_t n = (top_k > 0 && top_k < V) ? top_k + 1 : V;"),
    "top_p_exceeds_instead_of_reaches": ("if (cum >= target) {", "if (cum > target) {"),
    "top_p_not_renormalised_by_top_k": ("for (int64_t r = 0; r < n; ++r) mass_k += exp((order[r].z - m) / T);",
                                        "for (int64_t r = 0; r < V; ++r) mass_k += exp((order[r].z - m) / T);"),
    "truncated_target_not_renormalised": ("      if (n < 0) abort();\n      if (opt && opt->kept_tokens) opt->kept_tokens[trow0 + j] = n;",
                                          "      if (n < 0) abort();\n      lse_t[j] = oracle_row_lse(target, dtype, trow0 + j, V, T);\n"
                                          "      if (opt && opt->kept_tokens) opt->kept_tokens[trow0 + j] = n;"),
    "truncated_draft_not_renormalised": ("      if (n < 0) abort();\n      if (opt && opt->kept_tokens) opt->kept_tokens[n_t + drow0 + j] = n;",
                                         "      if (n < 0) abort();\n      lse_d[j] = oracle_row_lse(draft, dtype, drow0 + j, V, T);\n"
                                         "      if (opt && opt->kept_tokens) opt->kept_tokens[n_t + drow0 + j] = n;"),
    "ratio_ignores_target_cut": ("if (!kept(keep_t, j, V, x)) {\n      ratio = 0.0;", "if (0) {\n      ratio = 0.0;"),
    "bonus_from_untruncated_p": ("kind = ORACLE_TERM_BONUS;\n    for (int32_t v = 0; v < V; ++v)\n      w[v] = kept(keep_t, t, V, v) ?",
                                 "kind = ORACLE_TERM_BONUS;\n    for (int32_t v = 0; v < V; ++v)\n      w[v] = 1 ?"),
    "residual_from_untruncated_q": (": (kept(keep_d, t, V, v) ? exp(", ": (1 ? exp("),
    "invalid_top_p_accepted": ("top_p_milli < 0 || top_p_milli > 1000;", "top_p_milli < 0;"),
    # which Philox block and word each decision takes
    "draw_from_block_of_position_0": ("oracle_philox_block(seed, (uint32_t)i, (uint32_t)t, blk);\n    u = draw_uniform(blk);",
                                      "oracle_philox_block(seed, (uint32_t)i, 0u, blk);\n    u = draw_uniform(blk);"),
    "draw_from_word_2": ("return (double)(w[1] >> 8) / 16777216.0;", "return (double)(w[2] >> 8) / 16777216.0;"),
    "accept_from_block_of_next_position": ("oracle_philox_block(seed, (uint32_t)i, (uint32_t)j, blk);\n      r = accept_uniform(blk);",
                                           "oracle_philox_block(seed, (uint32_t)i, (uint32_t)(j + 1), blk);\n      r = accept_uniform(blk);"),
    "accept_from_word_3": ("return (double)((w[0] >> 8) + 1u) / 16777216.0;", "return (double)((w[3] >> 8) + 1u) / 16777216.0;"),
    "draw_counter_request_and_position_swapped": ("oracle_philox_block(seed, (uint32_t)i, (uint32_t)t, blk);\n    u = draw_uniform(blk);",
                                                  "oracle_philox_block(seed, (uint32_t)t, (uint32_t)i, blk);\n    u = draw_uniform(blk);"),
    # token trees
    "tree_residual_not_updated": ("          p[v] = p[v] > q[v] ? p[v] - q[v] : 0.0;\n          S += p[v];",
                                  "          S += p[v] > q[v] ? p[v] - q[v] : 0.0;"),
    "tree_residual_left_unnormalized": ("          for (int32_t v = 0; v < V; ++v) p[v] /= S_last;\n", ""),
    "tree_accept_block_of_depth": ("oracle_philox_block(seed, (uint32_t)i, (uint32_t)c, blk);",
                                   "oracle_philox_block(seed, (uint32_t)i, (uint32_t)a, blk);"),
    "tree_draw_block_of_node_index": ("oracle_philox_block(seed, (uint32_t)i, (uint32_t)row, blk);",
                                      "oracle_philox_block(seed, (uint32_t)i, (uint32_t)(row > 0 ? row - 1 : 0), blk);"),
    "tree_q_of_first_sibling": ("for (int32_t v = 0; v < V; ++v) q[v] = exp(logit_at(draft, dtype, qrow[c], V, v) / T - lse_d[c]);",
                                "for (int32_t v = 0; v < V; ++v) q[v] = exp(logit_at(draft, dtype, qrow[u + 1], V, v) / T - lse_d[u + 1]);"),
    "tree_stops_at_first_rejection": ("      for (int64_t c = u + 1; c < N && next < 0; ++c) {\n        if (parents[drow0 + c] != u) continue;",
                                      "      for (int64_t c = u + 1; c < N && next < 0 && !rejected; ++c) {\n        if (parents[drow0 + c] != u) continue;"),
    "tree_greedy_last_matching_child": ("      for (int64_t c = u + 1; c < N && next < 0; ++c) /* a child's index exceeds its parent's */",
                                        "      for (int64_t c = u + 1; c < N; ++c) /* a child's index exceeds its parent's */"),
    "tree_draft_row_index_ignored": ("qrow[n] = draft_row ? draft_row[drow0 + n] : drow0 + n;", "qrow[n] = drow0 + n < n_draft_rows ? drow0 + n : 0;"),
    "tree_parent_check_off_by_one": ("if (x < 0 || x >= V || par < -1 || par >= n ||", "if (x < 0 || x >= V || par < -1 || par > n ||"),
}


def _build_mutant(tmp_path, name):
    src = open(oracle.SOURCE).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    src = src.replace(old, new, 1)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    lib = str(tmp_path / f"lib{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", str(path), "-o", lib, "-lm"], check=True)
    return lib


def _pin_monte_carlo(lib_path, T=1.0):
    """Distinct rows per position, 60 calls x 4096 requests; fails if any chi-square p < 1e-6."""
    rng = np.random.default_rng(321)
    K, V, B = 3, 8, 4096
    zt = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
    zd = (zt[:K] + rng.standard_normal((K, V)) * 1.0).astype(np.float32)
    p = np.stack([exact.softmax(r, T) for r in zt])
    q = np.stack([exact.softmax(r, T) for r in zd])
    law = exact.round_distribution(p, q, grid=True)
    cu = offsets_from_depths(np.full(B, K))
    target, draft = np.tile(zt, (B, 1)), np.tile(zd, (B, 1))
    pmf = np.zeros(K + 1)
    reached = np.zeros((K + 1, V))
    for c in range(60):
        g = -np.log(-np.log(np.random.default_rng([5, c]).random((B * K, V))))
        tokens = np.argmax(draft.astype(np.float64) / T + g, axis=1).astype(np.int32)
        res = oracle.verify(target, draft, tokens, cu, T, 1000 + c, lib_path=lib_path)
        a = res["accepted_len"]
        if (a < 0).any():
            return False
        pmf += np.bincount(a, minlength=K + 1)
        slots = res["out_tokens"].reshape(B, K + 1)
        for j in range(K + 1):
            reached[j] += np.bincount(np.clip(slots[a >= j, j], 0, V - 1), minlength=V)
    pv = [stats.chisquare(pmf, law["pmf_accepted"] * pmf.sum()).pvalue]
    for j in range(K + 1):
        e = law["token_reached"][j] / law["token_reached"][j].sum() * reached[j].sum()
        if (reached[j][e == 0] > 0).any():
            return False
        pv.append(stats.chisquare(reached[j][e > 0], e[e > 0]).pvalue)
    return min(pv) > 1e-6


def _pin_lse(lib_path):
    lib = ctypes.CDLL(lib_path)
    lib.oracle_row_lse.restype = ctypes.c_double
    lib.oracle_row_lse.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_double]
    row = np.full(100, 3.0, dtype=np.float32)
    return abs(lib.oracle_row_lse(row.ctypes.data, 1, 0, 100, 0.5) - (6.0 + np.log(100))) < 1e-12


def _pin_greedy_tie(lib_path):
    row = np.zeros((2, 10), dtype=np.float32)
    row[0, [3, 6]] = 5.0
    res = oracle.verify(row, None, np.array([6], dtype=np.int32), offsets_from_depths([1]), 0.0, 0, lib_path=lib_path)
    return res["out_tokens"][0] == 3


def _pin_philox(lib_path, tmp_path):
    header = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not os.path.exists(header) or shutil.which("g++") is None:
        return True
    exe = str(tmp_path / "probe")
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(HERE, "rocrand_philox_probe.cpp"), "-o", exe], check=True)
    ref = subprocess.run([exe, "12345", "0", "4", "4"], check=True, capture_output=True, text=True).stdout
    lib = ctypes.CDLL(lib_path)
    lib.oracle_philox_block.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    got = []
    for i in range(4):
        for j in range(4):
            out = np.zeros(4, dtype=np.uint32)
            lib.oracle_philox_block(12345, i, j, out.ctypes.data)
            got.append(" ".join(f"{w:08x}" for w in out))
    return ref.split("\n")[:16] == got


def _pin_profiles(lib_path):
    """Request i of a batch with per-request (T_i, seed_i) equals request i of the scalar run with
    (T_i, seed_i); a NaN temperature rejects its request alone."""
    rng = np.random.default_rng(8)
    depths = rng.integers(0, 5, size=12)
    cu = offsets_from_depths(depths)
    n_d, B, V = int(cu[-1]), 12, 64
    target = (rng.standard_normal((n_d + B, V)) * 2).astype(np.float32)
    draft = (target[:n_d] + rng.standard_normal((n_d, V))).astype(np.float32)
    tokens = rng.integers(0, V, size=n_d).astype(np.int32)
    profiles = [(0.0, 3), (0.8, 4), (1.3, 5)]
    pick = np.arange(B) % 3
    T = np.array([profiles[k][0] for k in pick])
    T[7] = np.nan
    seeds = np.array([profiles[k][1] for k in pick], dtype=np.uint64)
    got = oracle.verify(target, draft, tokens, cu, T, seeds, lib_path=lib_path)
    if got["accepted_len"][7] != -1:
        return False
    for k, (t, sd) in enumerate(profiles):
        ref = oracle.verify(target, draft, tokens, cu, t, sd, lib_path=lib_path)
        for i in np.nonzero((pick == k) & (np.arange(B) != 7))[0]:
            lo, hi = cu[i] + i, cu[i + 1] + i + 1
            if got["accepted_len"][i] != ref["accepted_len"][i]:
                return False
            if not np.array_equal(got["out_tokens"][lo:hi], ref["out_tokens"][lo:hi]):
                return False
    return True


def _pin_stops(lib_path):
    """SDCP's example round with stops and budgets, and the caller-uniform special cases."""
    rows = np.zeros((4, 16), dtype=np.float32)
    for r, g in enumerate([7, 9, 13, 5]):
        rows[r, g] = 1.0
    toks, cu = np.array([7, 9, 11], dtype=np.int32), offsets_from_depths([3])
    for stop, budget, want in (([9], None, [7, 9]), ([13], None, [7, 9, 13]), ([], 1, [7]), ([], 2, [7, 9])):
        res = oracle.verify(rows, None, toks, cu, 0.0, 0, lib_path=lib_path, stop_lists=[stop],
                            budget=None if budget is None else [budget])
        n = int(res["emitted_len"][0])
        if res["out_tokens"][:n].tolist() != want or (res["out_tokens"][n:] != -1).any():
            return False
    # caller uniforms: r = 0 rejects exactly where p(x) = 0; the draw uses u of the drawn position
    rng = np.random.default_rng(5)
    target = rng.standard_normal((5, 12)).astype(np.float32)
    draft = (target[:4] + rng.standard_normal((4, 12))).astype(np.float32)
    tokens = rng.integers(0, 12, size=4).astype(np.int32)
    target[2, tokens[2]] = -np.inf
    u = np.array([0.1, 0.2, 0.999999, 0.4, 0.5])
    res = oracle.verify(target, draft, tokens, offsets_from_depths([4]), 1.0, 0, lib_path=lib_path,
                        accept_uniform=np.zeros(4), draw_uniform=u)
    if res["accepted_len"][0] != 2:
        return False
    w = np.maximum(exact.softmax(target[2], 1.0) - exact.softmax(draft[2], 1.0), 0.0)
    c = np.cumsum(w)
    if res["out_tokens"][2] != np.searchsorted(c, u[2] * c[-1], side="right"):
        return False
    # a budget of exactly a emits the accepted drafts and no extra token
    res = oracle.verify(target, draft, tokens, offsets_from_depths([4]), 1.0, 0, lib_path=lib_path,
                        accept_uniform=np.zeros(4), draw_uniform=u, budget=[2])
    return res["out_tokens"][:2].tolist() == tokens[:2].tolist() and (res["out_tokens"][2:] == -1).all()


def _pin_qrows(lib_path):
    """q rows equal to the rounded draft softmax: verdicts as the logit path's, up to near-ties."""
    from oracle.compare import compare_verdicts
    rng = np.random.default_rng(12)
    depths = rng.integers(1, 6, size=200)
    cu = offsets_from_depths(depths)
    n_d, B, V = int(cu[-1]), 200, 24
    target = (rng.standard_normal((n_d + B, V)) * 2).astype(np.float32)
    draft = (target[np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(B)])]
             + rng.standard_normal((n_d, V))).astype(np.float32)
    z = draft.astype(np.float64)
    q = np.exp(z - z.max(axis=1, keepdims=True))
    q = (q / q.sum(axis=1, keepdims=True)).astype(np.float32)
    g = -np.log(-np.log(rng.random((n_d, V))))
    tokens = np.argmax(z + g, axis=1).astype(np.int32)
    ref = oracle.verify(target, draft, tokens, cu, 1.0, 3, diag=True, lib_path=lib_path)
    got = oracle.verify(target, None, tokens, cu, 1.0, 3, draft_probs=q, lib_path=lib_path)
    return compare_verdicts(got["accepted_len"], got["out_tokens"], ref, cu, 1.0)["n_hard"] == 0


def _pin_filters(lib_path):
    """Every top-k / top-p pin of tests/filter_pins.py."""
    return all(check(lib_path) for check in filter_pins.ALL)


def _pin_keying(lib_path):
    """Every Philox keying pin of tests/keying_pins.py (block and word of each decision)."""
    return all(check(lib_path) for check in keying_pins.ALL)


def _pin_tree(lib_path):
    """Every token-tree pin of tests/tree_pins.py."""
    return all(check(lib_path) for check in tree_pins.ALL)


def test_unmutated_oracle_passes_every_pin(tmp_path):
    for check in (_pin_monte_carlo, _pin_lse, _pin_greedy_tie, _pin_profiles, _pin_stops, _pin_qrows, _pin_filters,
                  _pin_keying, _pin_tree):
        assert check(oracle.LIBRARY)
    assert _pin_philox(oracle.LIBRARY, tmp_path)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    oracle.load()  # make sure the reference build exists
    lib = _build_mutant(tmp_path, name)
    results = {
        "monte_carlo": _pin_monte_carlo(lib),
        "monte_carlo_T0.7": _pin_monte_carlo(lib, T=0.7),
        "lse": _pin_lse(lib),
        "greedy_tie": _pin_greedy_tie(lib),
        "philox": _pin_philox(lib, tmp_path),
        "profiles": _pin_profiles(lib),
        "stops_and_caller_uniforms": _pin_stops(lib),
        "qrows": _pin_qrows(lib),
        "top_k_top_p": _pin_filters(lib),
        "keying": _pin_keying(lib),
        "tree": _pin_tree(lib),
    }
    assert not all(results.values()), f"planted mistake {name!r} passed every pin: {results}"
