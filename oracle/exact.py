"""Brute-force exact output distribution of one speculative round on a tiny vocabulary.

TEST INFRASTRUCTURE ONLY.  This is a second, independent derivation of what the verification
step produces: instead of sampling, it sums over every draft tuple and every accept/reject branch,
so its results are exact probabilities (fp64, or Fractions when asked).  The tests use it to pin
the sampling oracle (Monte Carlo must match it) and check it against the closed forms that
"M7.8 - Speculative Serving" prints in sections 0x02 and 0x02B, and against the losslessness claim
of "SOTA-227" ("Why it is free rather than a trade") and SDCP Rule 2.

Model of a round (positions are "context-free": the target row p_j and draft row q_j of position j
do not depend on the tokens drafted before it, which is how the synthetic workloads are built):
  x_j ~ q_j independently; position j is accepted with probability min(1, p_j(x_j)/q_j(x_j)) given
  all earlier ones were; the first rejected position emits a token from normalize(max(p_j - q_j, 0));
  if all K are accepted the extra token comes from p_K.
With ``grid=True`` the accept test and the draw use the 2^-24 uniform grids that the verifier's
Philox words give (r = (k+1)/2^24, u = k/2^24), so the result is the exact law of the
implemented sampler rather than of the idealised one.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

GRID = 1 << 24


def softmax(z: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(z / T) in fp64."""
    a = np.asarray(z, dtype=np.float64) / temperature
    a = a - a.max()
    e = np.exp(a)
    return e / e.sum()


def _accept_probability(p: float, q: float, grid: bool) -> float:
    ratio = p / q
    if not grid:
        return min(1.0, ratio)
    # r = (k + 1) / 2^24 for k uniform in [0, 2^24): P(r <= ratio) = min(floor(ratio * 2^24), 2^24) / 2^24
    return min(np.floor(ratio * GRID), GRID) / GRID


def _draw_law(w: np.ndarray, grid: bool) -> np.ndarray:
    """Law of y = min{v : C(v) > u S} for u uniform on [0,1) (or on the 2^-24 grid)."""
    S = w.sum()
    if not grid:
        return w / S
    # y = v exactly for the grid points k with C(v-1) <= (k/2^24) S < C(v)
    C = np.concatenate([[0.0], np.cumsum(w)])
    # number of k in [0, 2^24) with k < C(v) * 2^24 / S is ceil(C(v) * 2^24 / S), clipped
    cnt = np.minimum(np.ceil(C * GRID / S), GRID)
    return np.diff(cnt) / GRID


def round_distribution(p_rows: np.ndarray, q_rows: np.ndarray, grid: bool = False) -> dict:
    """Exact law of one round by enumeration over all V^K draft tuples.

    p_rows: (K+1, V) target distributions; q_rows: (K, V) draft distributions.
    Returns:
      pmf_accepted  (K+1,)     P(A = a)
      token_reached (K+1, V)   P(position j emits token v and is reached), so that
                               token_reached[j] / token_reached[j].sum() = P(y_j = v | C > j)
      first_token   (V,)       P(y_0 = v)
    """
    p_rows = np.asarray(p_rows, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    K = q_rows.shape[0]
    V = p_rows.shape[1]
    assert p_rows.shape == (K + 1, V)
    pmf = np.zeros(K + 1)
    reached = np.zeros((K + 1, V))
    resid = []
    for j in range(K):
        w = np.maximum(p_rows[j] - q_rows[j], 0.0)
        resid.append(_draw_law(w, grid) if w.sum() > 0 else _draw_law(p_rows[j], grid))
    bonus = _draw_law(p_rows[K], grid)
    for xs in itertools.product(range(V), repeat=K):
        weight = 1.0
        for j, x in enumerate(xs):
            weight *= q_rows[j][x]
        if weight == 0.0:
            continue
        alive = weight  # probability of this tuple and of reaching position j with all earlier accepted
        for j, x in enumerate(xs):
            acc = _accept_probability(p_rows[j][x], q_rows[j][x], grid)
            pmf[j] += alive * (1.0 - acc)
            reached[j] += alive * (1.0 - acc) * resid[j]
            reached[j][x] += alive * acc
            alive *= acc
        pmf[K] += alive
        reached[K] += alive * bonus
    return {"pmf_accepted": pmf, "token_reached": reached, "first_token": reached[0].copy()}


def round_distribution_fraction(p_rows, q_rows) -> dict:
    """The same enumeration in exact rational arithmetic (inputs given as Fractions or ints)."""
    p_rows = [[Fraction(v) for v in row] for row in p_rows]
    q_rows = [[Fraction(v) for v in row] for row in q_rows]
    K = len(q_rows)
    V = len(p_rows[0])
    pmf = [Fraction(0)] * (K + 1)
    reached = [[Fraction(0)] * V for _ in range(K + 1)]
    resid = []
    for j in range(K):
        w = [max(p_rows[j][v] - q_rows[j][v], Fraction(0)) for v in range(V)]
        S = sum(w)
        resid.append([wv / S for wv in w] if S > 0 else list(p_rows[j]))
    for xs in itertools.product(range(V), repeat=K):
        alive = Fraction(1)
        for j, x in enumerate(xs):
            alive *= q_rows[j][x]
        if alive == 0:
            continue
        for j, x in enumerate(xs):
            acc = min(Fraction(1), p_rows[j][x] / q_rows[j][x])
            pmf[j] += alive * (1 - acc)
            for v in range(V):
                reached[j][v] += alive * (1 - acc) * resid[j][v]
            reached[j][x] += alive * acc
            alive *= acc
        pmf[K] += alive
        for v in range(V):
            reached[K][v] += alive * p_rows[K][v]
    return {"pmf_accepted": pmf, "token_reached": reached}


def acceptance_rate(p: np.ndarray, q: np.ndarray) -> float:
    """alpha = sum_v min(p(v), q(v)): the probability that a token drawn from q is accepted."""
    return float(np.minimum(p, q).sum())
