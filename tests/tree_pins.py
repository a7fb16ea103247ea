"""Pins of the oracle's token-tree verification (oracle_verify_tree), usable against a mutated build.

TEST INFRASTRUCTURE ONLY.  The rule is multi-step speculative sampling over a token tree (Miao et
al., "SpecInfer: Accelerating Large Language Model Serving with Tree-based Speculative Inference and
Verification", ASPLOS 2024, section 4), and on trees at T = 0 the greedy rule of "Speculative
Decoding Coordination Protocol (SDCP)", section "Acceptance Rules", Rule 1.  What pins it, none of
it computed by the oracle:

  * hand-worked trees whose every decision is forced (tests/golden/tree_verification.json);
  * a chain of nodes is a linear draft: the tree walk must give the linear oracle's verdicts, which
    are pinned on their own (the exact law, the keying pins, the planted mistakes);
  * at T = 0, random trees against a walk written here in numpy (the first child equal to the
    target argmax);
  * losslessness, the property the method exists for: with sibling tokens drawn independently from
    the drafter's distribution at their parent's context and target rows that depend on the context
    only, the emitted tokens follow the target's autoregressive law; chi-square tests of the first,
    second and third emitted token given the tokens before them;
  * the uniforms of a tree: a second child's accept decision placed within 2^-24 of r from the
    Philox block of its own node index, and a residual draw below the root with u from the block of
    its target row, both computed here from the rocRAND-pinned Philox.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy import stats

import keying_pins as KP
from oracle import oracle
from workloads import offsets_from_depths

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tree_verification.json")


def _rows(x):
    return np.array([[-np.inf if v == "-inf" else float(v) for v in r] for r in x], dtype=np.float32)


def pin_hand_worked(lib_path: str = oracle.LIBRARY) -> bool:
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        n = len(case["tokens"])
        draft = None if case["draft"] is None else _rows(case["draft"])
        res = oracle.verify_tree(_rows(case["target"]), draft, case["tokens"], case["parents"],
                                 offsets_from_depths([n]), case["T"], 17, diag=True, lib_path=lib_path)
        if (res["accepted_len"][0] != case["accepted_len"] or res["out_tokens"].tolist() != case["out_tokens"]
                or res["accepted_nodes"].tolist() != case["accepted_nodes"]
                or res["terminal_kind"][0] != case["terminal_kind"]):
            return False
    b = g["bad_requests"]
    res = oracle.verify_tree(_rows(b["target"]), _rows(b["draft"]), b["tokens"], b["parents"],
                             offsets_from_depths(b["depths"]), b["T"], 3, lib_path=lib_path)
    return (res["accepted_len"].tolist() == b["accepted_len"] and res["out_tokens"].tolist() == b["out_tokens"]
            and res["accepted_nodes"].tolist() == b["accepted_nodes"])


def pin_chain_equals_linear(lib_path: str = oracle.LIBRARY) -> bool:
    rng = np.random.default_rng(81)
    for T, dtype in ((1.0, np.float32), (0.6, np.float32), (0.0, np.float32), (1.0, np.uint16)):
        depths = rng.integers(0, 9, size=96)
        cu = offsets_from_depths(depths)
        B, n, V = len(depths), int(cu[-1]), 300
        target = (rng.standard_normal((n + B, V)) * 2.0).astype(np.float32)
        t_of_d = np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(B)]).astype(int)
        draft = (target[t_of_d] + rng.standard_normal((n, V)) * rng.uniform(0.3, 2.0, size=(n, 1))).astype(np.float32)
        if dtype == np.uint16:  # bf16 bits: the top half of each binary32
            target = (target.view(np.uint32) >> 16).astype(np.uint16)
            draft = (draft.view(np.uint32) >> 16).astype(np.uint16)
        tokens = rng.integers(0, V, size=n).astype(np.int32)
        parents = np.concatenate([np.arange(-1, k - 1) for k in depths]).astype(np.int32)
        seed = int(rng.integers(0, 2**63))
        lin = oracle.verify(target, draft if T > 0 else None, tokens, cu, T, seed, diag=True, lib_path=lib_path)
        tree = oracle.verify_tree(target, draft if T > 0 else None, tokens, parents, cu, T, seed, diag=True,
                                  lib_path=lib_path)
        if not (np.array_equal(lin["accepted_len"], tree["accepted_len"])
                and np.array_equal(lin["out_tokens"], tree["out_tokens"])
                and np.array_equal(lin["terminal_kind"], tree["terminal_kind"])):
            return False
        if T > 0 and not np.array_equal(lin["resid_mass"], tree["resid_mass"]):
            return False
        for i, a in enumerate(lin["accepted_len"]):
            want = list(range(a)) + [-1] * (int(depths[i]) - a)
            if tree["accepted_nodes"][cu[i]:cu[i + 1]].tolist() != want:
                return False
    return True


def _random_trees(rng, B, max_nodes):
    """B random trees in node order (each parent an earlier node or the root)."""
    sizes = rng.integers(0, max_nodes + 1, size=B)
    parents = [np.array([rng.integers(-1, k) for k in range(s)], dtype=np.int32) for s in sizes]
    return sizes, parents


def pin_greedy_brute_force(lib_path: str = oracle.LIBRARY) -> bool:
    rng = np.random.default_rng(82)
    B, V = 200, 6
    sizes, parents = _random_trees(rng, B, 12)
    cu = offsets_from_depths(sizes)
    n = int(cu[-1])
    target = rng.integers(0, 3, size=(n + B, V)).astype(np.float32)  # many ties
    tokens = rng.integers(0, V, size=n).astype(np.int32)
    res = oracle.verify_tree(target, None, tokens, np.concatenate(parents), cu, 0.0, 0, lib_path=lib_path)
    for i in range(B):
        par, tok = parents[i], tokens[cu[i]:cu[i + 1]]
        u, path = -1, []
        while True:
            g = int(np.argmax(target[cu[i] + i + u + 1]))  # numpy's argmax: the first maximum
            match = [c for c in range(sizes[i]) if par[c] == u and tok[c] == g]
            if not match:
                break
            u = match[0]
            path.append(u)
        want = [int(tok[c]) for c in path] + [g] + [-1] * (sizes[i] - len(path))
        if res["accepted_len"][i] != len(path) or res["out_tokens"][cu[i] + i: cu[i + 1] + i + 1].tolist() != want:
            return False
        if res["accepted_nodes"][cu[i]:cu[i + 1]].tolist() != path + [-1] * (sizes[i] - len(path)):
            return False
    return True


def _softmax(z, T):
    z = np.asarray(z, dtype=np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def pin_lossless(lib_path: str = oracle.LIBRARY, T: float = 1.0, calls: int = 40) -> bool:
    """Root with three children, each with two: nine nodes per request.  Target rows depend on the
    token path (the context) only, draft rows on the parent's context; siblings are drawn
    independently from their parent context's draft distribution.  The first emitted token must
    follow p(root), the second p(v) given a first accepted token v, the third p(v, w)."""
    rng = np.random.default_rng(83)
    V, B = 4, 4096
    ctx = [()] + [(v,) for v in range(V)] + [(v, w) for v in range(V) for w in range(V)]
    zp = {c: (rng.standard_normal(V) * 1.2).astype(np.float32) for c in ctx}
    zq = {c: (zp[c] + rng.standard_normal(V) * 0.9).astype(np.float32) for c in ctx if len(c) < 2}
    parents = np.array([-1, -1, -1, 0, 0, 1, 1, 2, 2], dtype=np.int32)
    N = len(parents)
    cu = offsets_from_depths(np.full(B, N))
    counts = {c: np.zeros(V) for c in ctx}
    for call in range(calls):
        g = np.random.default_rng([84, call])
        tok = np.zeros((B, N), dtype=np.int32)
        q0 = _softmax(zq[()], T)
        tok[:, :3] = g.choice(V, size=(B, 3), p=q0)
        for n in range(3, N):
            par_tok = tok[:, parents[n]]
            for v in range(V):
                sel = par_tok == v
                tok[sel, n] = g.choice(V, size=int(sel.sum()), p=_softmax(zq[(v,)], T))
        target = np.zeros((B * (N + 1), V), dtype=np.float32)
        draft = np.zeros((B * N, V), dtype=np.float32)
        for i in range(B):
            t0, d0 = i * (N + 1), i * N
            target[t0] = zp[()]
            for n in range(N):
                path = (int(tok[i, n]),) if parents[n] < 0 else (int(tok[i, parents[n]]), int(tok[i, n]))
                target[t0 + n + 1] = zp[path]
                draft[d0 + n] = zq[path[:-1]]
        res = oracle.verify_tree(target, draft, tok.reshape(-1), np.tile(parents, B), cu, T, 9000 + call,
                                 lib_path=lib_path)
        a = res["accepted_len"]
        if (a < 0).any():
            return False
        out = res["out_tokens"].reshape(B, N + 1)
        for i in range(B):
            prefix = ()
            for d in range(int(a[i]) + 1):
                counts[prefix][out[i, d]] += 1
                prefix = prefix + (int(out[i, d]),)
    pvals = []
    for c in ctx:
        m = counts[c].sum()
        if m < 200:
            continue
        e = _softmax(zp[c], T) * m
        pvals.append(stats.chisquare(counts[c], e).pvalue)
    return len(pvals) >= 10 and min(pvals) > 1e-6


def pin_tree_keying(lib_path: str = oracle.LIBRARY, seed: int = 0x7EE5) -> bool:
    # (a) the second child's accept test takes r from the block of its own node index
    B, V = 64, 8
    cu = offsets_from_depths(np.full(B, 2))
    target = np.zeros((3 * B, V), dtype=np.float32)
    draft = np.zeros((2 * B, V), dtype=np.float32)
    tokens = np.zeros(2 * B, dtype=np.int32)
    parents = np.full(2 * B, -1, dtype=np.int32)
    expect, used = [], []
    for i in range(B):
        t0, d0 = 3 * i, 2 * i
        target[t0, 7] = -np.inf  # p(7) = 0 at the root ...
        draft[d0, :7] = -np.inf  # ... and node 0 proposes 7 with q = 1: rejected, residual = p
        tokens[d0] = 7
        x = i % 7
        tokens[d0 + 1] = x  # node 1 against an all-zero draft row: q = 1/8
        r = KP._accept_r(seed, i, 1)
        lo, hi = (r, r + KP.GRID) if (i // 7) % 2 == 0 else (r - KP.GRID, r)
        rho = 0.5 * (lo + hi)  # 8 e^d / (e^d + 6) = rho
        d = np.float32(np.log(6.0 * rho / (8.0 - rho)))
        ratio = 8.0 * np.exp(np.float64(d)) / (np.exp(np.float64(d)) + 6.0)
        target[t0, x] = d
        used.append(abs(ratio - r) > 1e-10)
        expect.append(1 if r <= ratio else 0)
    res = oracle.verify_tree(target, draft, tokens, parents, cu, 1.0, seed, lib_path=lib_path)
    got = res["accepted_len"]
    if any(u and got[i] != expect[i] for i, u in enumerate(used)) or sum(used) < B // 2:
        return False
    # (b) a residual draw below the root takes u from the block of its target row
    rng = np.random.default_rng(85)
    B, V = 48, 1000
    cu = offsets_from_depths(np.full(B, 2))
    target = (rng.standard_normal((3 * B, V)) * 2.0).astype(np.float32)
    draft = (rng.standard_normal((2 * B, V)) * 2.0).astype(np.float32)
    tokens = rng.integers(0, V, size=2 * B).astype(np.int32)
    parents = np.tile(np.array([-1, 0], dtype=np.int32), B)
    for i in range(B):
        t0, d0 = 3 * i, 2 * i
        draft[d0] = target[t0]  # node 0 accepted: its row equals the root's
        target[t0 + 1, tokens[d0 + 1]] = -30.0  # node 1 rejected: p(x) tiny, q(x) large
        draft[d0 + 1, tokens[d0 + 1]] = 30.0
    res = oracle.verify_tree(target, draft, tokens, parents, cu, 1.0, seed, lib_path=lib_path)
    if res["accepted_len"].tolist() != [1] * B:
        return False
    for i in range(B):
        w = np.maximum(_softmax(target[3 * i + 1], 1.0) - _softmax(draft[2 * i + 1], 1.0), 0.0)
        y, margin = KP._categorical(w, KP._draw_u(seed, i, 1))
        if margin > 1e-9 and res["out_tokens"][3 * i + 1] != y:
            return False
    return True


def shared_rows(b):
    """The batch's per-node draft rows folded to one row per parent context: (rows, draft_row)."""
    req = np.repeat(np.arange(b.B), np.diff(b.cu))
    ctx = b.cu[req] + req + b.parents + 1  # each node's parent context, as a target row index
    keys, first, draft_row = np.unique(ctx, return_index=True, return_inverse=True)
    return np.ascontiguousarray(b.draft[first]), draft_row.astype(np.int32)


def pin_shared_draft_rows(lib_path: str = oracle.LIBRARY) -> bool:
    """Siblings that share one draft row by index give the verdicts (and diagnostics) of the same
    tree with a copy of that row per node; an index outside the rows rejects its request alone."""
    from workloads import make_tree
    for T, kind in ((1.0, "random"), (0.8, "kary"), (0.0, "star")):
        rng = np.random.default_rng(86)
        b = make_tree("shared", rng.integers(0, 20, size=40), kind, 200, "fp32", T, 2.0, 1.0, data_seed=87,
                      verify_seed=3)
        draft = b.draft if T > 0 else np.zeros((b.n_draft_rows, b.V), np.float32)
        rows, idx = shared_rows(type(b)(**{**b.__dict__, "draft": draft}))
        if T > 0 and rows.shape[0] >= b.n_draft_rows:
            return False  # the batch must actually share rows
        full = oracle.verify_tree(b.target, b.draft, b.tokens, b.parents, b.cu, T, 5, diag=True, lib_path=lib_path)
        comp = oracle.verify_tree(b.target, rows if T > 0 else None, b.tokens, b.parents, b.cu, T, 5, diag=True,
                                  lib_path=lib_path, draft_row=idx)
        for k in ("accepted_len", "out_tokens", "accepted_nodes", "terminal_kind"):
            if not np.array_equal(full[k], comp[k]):
                return False
        for k in ("ratio", "resid_mass", "draft_lse"):
            if not np.array_equal(full[k], comp[k], equal_nan=True):
                return False
        if T > 0:
            bad = idx.copy()
            i = int(np.argmax(np.diff(b.cu) > 0))  # a request with nodes
            bad[b.cu[i]] = rows.shape[0]
            res = oracle.verify_tree(b.target, rows, b.tokens, b.parents, b.cu, T, 5, lib_path=lib_path, draft_row=bad)
            others = np.arange(b.B) != i
            if res["accepted_len"][i] != -1 or not np.array_equal(res["accepted_len"][others],
                                                                   full["accepted_len"][others]):
                return False
    return True


ALL = (pin_hand_worked, pin_chain_equals_linear, pin_greedy_brute_force, pin_lossless, pin_tree_keying,
       pin_shared_draft_rows)
