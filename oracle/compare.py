"""GPU-vs-oracle verdict comparison with first-divergence attribution.

TEST INFRASTRUCTURE ONLY.  A request's verdict (accepted length and emitted tokens) must equal the
oracle's exactly.  The only excuse is a first divergence at a decision the oracle itself took
within ``eps`` of its threshold: an accept test with |r - p/q| < eps, an extra-token draw whose
CDF margin is below eps, or (top-p) a row of the request whose nucleus cut lies within eps of its
threshold, relative to the row's top-k mass (there the kept set itself may differ by one rank, and
every probability of the row with it).  Greedy verdicts have no excuse.
"""
from __future__ import annotations

import numpy as np


def compare_verdicts(acc_gpu, out_gpu, ref: dict, cu, temperature, eps: float = 1e-6) -> dict:
    """ref: oracle.verify(..., diag=True); temperature: the batch's, or one per request.  Returns
    counts and the list of hard mismatches."""
    acc_gpu = np.asarray(acc_gpu)
    out_gpu = np.asarray(out_gpu)
    cu = np.asarray(cu)
    acc_ref, out_ref = ref["accepted_len"], ref["out_tokens"]
    B = acc_ref.shape[0]
    hard, excused = [], []
    for i in range(B):
        K = int(cu[i + 1] - cu[i])
        if acc_ref[i] == -1 and not (0 <= K <= 64 and cu[i] >= 0 and cu[i + 1] <= out_ref.shape[0] - B):
            if acc_gpu[i] != -1:
                hard.append((i, "invalid request not rejected"))
            continue
        s = slice(int(cu[i]) + i, int(cu[i]) + i + K + 1)
        if acc_gpu[i] == acc_ref[i] and np.array_equal(out_gpu[s], out_ref[s]):
            continue
        t_i = temperature[i] if np.ndim(temperature) else temperature
        fm = ref.get("filter_margin")
        if t_i != 0 and fm is not None:
            # a cut that moves by one rank can also decide whether a draft token is kept at all
            n_t = out_ref.shape[0]
            rows = list(range(int(cu[i]) + i, int(cu[i]) + i + K + 1))
            rows += [n_t + int(cu[i]) + j for j in range(K) if n_t + int(cu[i]) + j < fm.shape[0]]
            closest = float(np.min(fm[rows]))
            if closest < eps:
                excused.append((i, f"top-p cut at relative margin {closest:.3g}"))
                continue
        if t_i == 0 or acc_ref[i] == -1 or acc_gpu[i] == -1:
            hard.append((i, f"accepted {acc_gpu[i]} vs {acc_ref[i]}"))
            continue
        a_g, a_r = int(acc_gpu[i]), int(acc_ref[i])
        if a_g != a_r:
            j = min(a_g, a_r)  # the first position whose accept decision differs
            margin = ref["accept_margin"][int(cu[i]) + j]
            what = f"accept decision at position {j}, oracle margin {margin:.3g}"
        else:
            prefix_ok = np.array_equal(out_gpu[s][:a_r], out_ref[s][:a_r]) and (out_gpu[s][a_r + 1:] == -1).all()
            margin = ref["cdf_margin"][i] if prefix_ok else np.inf
            what = f"drawn token {out_gpu[s][a_r]} vs {out_ref[s][a_r]}, oracle CDF margin {margin:.3g}"
        (excused if margin < eps else hard).append((i, what))
    return {"requests": B, "hard": hard, "excused": excused, "n_hard": len(hard), "n_excused": len(excused)}


def compare_tree_verdicts(acc_gpu, out_gpu, nodes_gpu, ref: dict, cu, parents, temperature,
                          eps: float = 1e-6) -> dict:
    """Token trees.  ref: oracle.verify_tree(..., diag=True).  A request must match the oracle's
    accepted depth, path (accepted_nodes) and tokens exactly; the only excuse is a first divergence
    at a decision the oracle took within eps of its threshold: an accept test of a child of the last
    common node (|r - ratio| < eps at a child the oracle tested there), or, with equal paths, the
    extra token's draw (CDF margin < eps).  Greedy trees have no excuse."""
    acc_gpu, out_gpu, nodes_gpu = np.asarray(acc_gpu), np.asarray(out_gpu), np.asarray(nodes_gpu)
    cu, parents = np.asarray(cu), np.asarray(parents)
    acc_ref, out_ref, nodes_ref = ref["accepted_len"], ref["out_tokens"], ref["accepted_nodes"]
    B = acc_ref.shape[0]
    hard, excused = [], []
    for i in range(B):
        lo, hi = int(cu[i]), int(cu[i + 1])
        N = hi - lo
        if acc_ref[i] == -1 and not (0 <= N <= 64 and lo >= 0 and hi <= nodes_ref.shape[0]):
            if acc_gpu[i] != -1:
                hard.append((i, "invalid request not rejected"))
            continue
        s = slice(lo + i, hi + i + 1)
        if (acc_gpu[i] == acc_ref[i] and np.array_equal(out_gpu[s], out_ref[s])
                and np.array_equal(nodes_gpu[lo:hi], nodes_ref[lo:hi])):
            continue
        if temperature == 0 or acc_ref[i] == -1 or acc_gpu[i] == -1:
            hard.append((i, f"accepted {acc_gpu[i]} vs {acc_ref[i]}"))
            continue
        a_g, a_r = int(acc_gpu[i]), int(acc_ref[i])
        pg, pr = nodes_gpu[lo:lo + a_g].tolist(), nodes_ref[lo:lo + a_r].tolist()
        d = 0
        while d < min(a_g, a_r) and pg[d] == pr[d]:
            d += 1
        if d < max(a_g, a_r):  # the walks part at depth d: an accept test among the children of the common node
            u = pr[d - 1] if d > 0 else -1
            kids = [lo + c for c in range(N) if parents[lo + c] == u]
            m = ref["accept_margin"][kids]
            margin = float(np.nanmin(m)) if np.isfinite(m).any() else np.inf
            what = f"paths part at depth {d} (node {u}), smallest oracle accept margin there {margin:.3g}"
        else:
            margin = ref["cdf_margin"][i]
            what = f"drawn token {out_gpu[s][a_r]} vs {out_ref[s][a_r]}, oracle CDF margin {margin:.3g}"
        (excused if margin < eps else hard).append((i, what))
    return {"requests": B, "hard": hard, "excused": excused, "n_hard": len(hard), "n_excused": len(excused)}
