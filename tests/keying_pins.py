"""Pins of the oracle's uniform keying at positions past the first, usable against a mutated build.

TEST INFRASTRUCTURE ONLY.  SDCP ("Speculative Decoding Coordination Protocol (SDCP)", section
"Acceptance Rules", Rule 2) takes one uniform per position and purpose; the verifier's uniforms come
from the Philox4x32-10 block keyed by the seed with counter (position j, request i, 0, 0): word 0
gives the accept test r = ((w0 >> 8) + 1) 2^-24, word 1 the draw u = (w1 >> 8) 2^-24 of the extra
token, taken from the block of the position the token is drawn at.  The Philox function itself is
pinned word for word against rocRAND's generator (test_oracle_philox.py); these pins fix which
block and which word each decision takes, with every expected value computed here from the stored
logits in numpy:

  * forced bonus: draft rows equal to the target rows give p/q = 1 at every position, so every
    draft is accepted and the bonus at t = K_i is the categorical draw from p_K by
    searchsorted(cumsum(p_K), u S, side="right") with u from block (i, K_i);
  * forced rejection at t: equal rows before t, and at t the drafted token's logit is -30 in the
    target row and +30 in the draft row, so p/q < 2^-24 <= r; the correction is the same
    searchsorted over cumsum(max(p_t - q_t, 0)) with u from block (i, t);
  * accept decisions on the edge: at position j the ratio is placed half a 2^-24 step above or
    below r from block (i, j), word 0 (rows equal elsewhere), so a decision that takes r from any
    other block or word flips about half of the requests.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle
from workloads import offsets_from_depths

GRID = 2.0 ** -24


def _softmax(z, T):
    z = np.asarray(z, dtype=np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def _accept_r(seed, i, j):
    return ((int(oracle.philox_block(seed, i, j)[0]) >> 8) + 1) * GRID


def _draw_u(seed, i, t):
    return (int(oracle.philox_block(seed, i, t)[1]) >> 8) * GRID


def _categorical(w, u):
    """searchsorted(cumsum(w), u S, side="right") and its CDF margin (distance of u to a step)."""
    c = np.cumsum(w)
    S = c[-1]
    y = int(np.searchsorted(c, u * S, side="right"))
    lo = (c[y - 1] if y > 0 else 0.0) / S
    return y, min(u - lo, c[y] / S - u)


def pin_forced_bonus(lib_path: str = oracle.LIBRARY, T: float = 1.0, seed: int = 0x5EED0B0) -> bool:
    rng = np.random.default_rng(71)
    depths = np.array([1, 2, 3, 4, 5, 6, 3, 3] * 6)
    B, V = len(depths), 1000
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    target = (rng.standard_normal((n_d + B, V)) * 2.0).astype(np.float32)
    t_of_d = np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(B)]).astype(int)
    draft = np.ascontiguousarray(target[t_of_d])
    tokens = rng.integers(0, V, size=n_d).astype(np.int32)
    res = oracle.verify(target, draft, tokens, cu, T, seed, lib_path=lib_path)
    if res["accepted_len"].tolist() != depths.tolist():
        return False
    for i, K in enumerate(depths):
        y, margin = _categorical(_softmax(target[cu[i] + i + K], T), _draw_u(seed, i, int(K)))
        if margin > 1e-9 and res["out_tokens"][cu[i] + i + K] != y:
            return False
    return True


def pin_forced_rejection(lib_path: str = oracle.LIBRARY, T: float = 1.0, seed: int = 0xC0FFEE) -> bool:
    rng = np.random.default_rng(72)
    B, K, V = 48, 4, 1000
    depths = np.full(B, K)
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    target = (rng.standard_normal((n_d + B, V)) * 2.0).astype(np.float32)
    t_of_d = np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(B)]).astype(int)
    draft = np.ascontiguousarray(target[t_of_d])
    tokens = rng.integers(0, V, size=n_d).astype(np.int32)
    reject_at = np.arange(B) % K  # the rejected position of each request: every t < K in turn
    for i in range(B):
        t = int(reject_at[i])
        x = tokens[cu[i] + t]
        target[cu[i] + i + t, x] = -30.0
        draft[cu[i] + t, x] = 30.0
    res = oracle.verify(target, draft, tokens, cu, T, seed, lib_path=lib_path)
    if res["accepted_len"].tolist() != reject_at.tolist():
        return False
    for i in range(B):
        t = int(reject_at[i])
        w = np.maximum(_softmax(target[cu[i] + i + t], T) - _softmax(draft[cu[i] + t], T), 0.0)
        y, margin = _categorical(w, _draw_u(seed, i, t))
        if margin > 1e-9 and res["out_tokens"][cu[i] + i + t] != y:
            return False
    return True


def _edge_logit(r, above: bool):
    """A binary32 logit delta whose ratio 8 e^delta / (7 + e^delta) (token x of an 8-token row whose
    other logits are 0, against an all-zero draft row) lies strictly inside (r, r + 2^-24) when
    above, else inside (r - 2^-24, r)."""
    lo, hi = (r, r + GRID) if above else (r - GRID, r)
    rho = 0.5 * (lo + hi)
    d = np.float32(np.log(7.0 * rho / (8.0 - rho)))
    for _ in range(64):
        ratio = 8.0 * np.exp(np.float64(d)) / (7.0 + np.exp(np.float64(d)))
        if lo < ratio < hi:
            return d, ratio
        d = np.nextafter(d, np.float32(np.inf) if ratio <= lo else np.float32(-np.inf), dtype=np.float32)
    raise AssertionError("no binary32 logit places the ratio inside the window")


def pin_accept_edges(lib_path: str = oracle.LIBRARY, seed: int = 0xED6E5) -> bool:
    B, K, V = 64, 4, 8
    depths = np.full(B, K)
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    target = np.zeros((n_d + B, V), dtype=np.float32)
    draft = np.zeros((n_d, V), dtype=np.float32)
    tokens = ((np.arange(n_d) * 3) % V).astype(np.int32)
    expect = []
    for i in range(B):
        j = i % K
        r = _accept_r(seed, i, j)
        above = (i // K) % 2 == 0
        d, ratio = _edge_logit(r, above)
        target[cu[i] + i + j, tokens[cu[i] + j]] = d
        expect.append(K if r <= ratio else j)  # equal rows elsewhere: p/q = 1, always accepted
    res = oracle.verify(target, draft, tokens, cu, 1.0, seed, lib_path=lib_path)
    return res["accepted_len"].tolist() == expect


ALL = (pin_forced_bonus, pin_forced_rejection, pin_accept_edges)
