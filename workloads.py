"""Seeded synthetic workloads for the verification step.

Shared by the oracle tests, the GPU parity tests, the smoke check and the benchmark.  It draws
inputs only: logits, ragged depths and the drafter's tokens.  It holds none of the verifier's
arithmetic: draft tokens are drawn with the Gumbel-max trick (x = argmax_v z_v/T + G_v), which the
verification step never uses, and at temperature 0 the drafter proposes its own argmax.

The pages measure on no public benchmark or dataset that could be loaded here.  Their serving
workloads and trained models are replaced by Gaussian logits: target z ~ N(0, s_t^2), draft
z + N(0, s_d^2), so that the draft/target agreement (the acceptance rate alpha) is set by s_d.

Layout of a ragged batch ("M7.8 - Speculative Serving", section 0x00, background on the serving unit: N_query = sum_i (K_i + 1)):
  cu[i]       exclusive prefix sum of the depths K_i, cu[0] = 0, cu[B] = n_draft_rows
  draft rows  request i, position j < K_i  -> row cu[i] + j
  target rows request i, position j <= K_i -> row cu[i] + i + j
bf16 logits are kept as their raw 16 bits (uint16), rounded to nearest-even from fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + (((b >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Batch:
    """One verification call's inputs, host side."""
    name: str
    V: int
    dtype: str                    # "bf16" or "fp32"
    temperature: float
    seed: int                     # the verifier's seed
    target: np.ndarray            # (n_draft_rows + B, V) uint16 bf16 bits or float32
    draft: np.ndarray | None      # (n_draft_rows, V), None for greedy workloads
    tokens: np.ndarray            # (n_draft_rows,) int32
    cu: np.ndarray                # (B + 1,) int32
    meta: dict = field(default_factory=dict)
    temp_each: np.ndarray | None = None  # (B,) float32: one temperature per request, else None
    seed_each: np.ndarray | None = None  # (B,) uint64: one seed per request (with temp_each)
    qrows: np.ndarray | None = None      # (n_draft_rows, V) float32 draft distributions, else None
    top_k: np.ndarray | None = None      # (B,) int32 top-k of each request's profile, else None
    top_p_milli: np.ndarray | None = None  # (B,) int32 top-p in thousandths, else None
    parents: np.ndarray | None = None    # (n_draft_rows,) int32: token trees, each node's parent (-1: root)
    draft_row: np.ndarray | None = None  # (n_draft_rows,) int32: token trees, each node's draft row (shared rows)

    @property
    def B(self) -> int:
        return int(self.cu.shape[0] - 1)

    @property
    def n_draft_rows(self) -> int:
        return int(self.tokens.shape[0])

    @property
    def depths(self) -> np.ndarray:
        return np.diff(self.cu)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def algorithmic_bytes(self) -> int:
        """Every logit the method needs, read once: target rows, plus the draft rows of every request
        that samples (T > 0)."""
        if self.qrows is not None:  # the draft side is read where it is needed, counted per call
            draft_rows = 0
        elif self.temp_each is not None:
            draft_rows = int(np.sum(self.depths[self.temp_each > 0]))
        else:  # token trees may share draft rows among siblings
            given = self.draft.shape[0] if self.draft is not None and self.draft_row is not None else self.n_draft_rows
            draft_rows = given if self.temperature > 0 else 0
        return (self.target.shape[0] + draft_rows) * self.V * self.elem_bytes

    def target_f32(self) -> np.ndarray:
        return bf16_to_f32(self.target) if self.dtype == "bf16" else self.target

    def draft_f32(self) -> np.ndarray | None:
        if self.draft is None:
            return None
        return bf16_to_f32(self.draft) if self.dtype == "bf16" else self.draft


def offsets_from_depths(depths) -> np.ndarray:
    d = np.asarray(depths, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(d)]).astype(np.int32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def _gumbel_tokens(rng: np.random.Generator, stored_draft: np.ndarray, dtype: str, temperature: float,
                   block_rows: int = 64) -> np.ndarray:
    """Draft tokens x_j ~ softmax(stored draft row / T) via x = argmax(z/T + Gumbel)."""
    n, V = stored_draft.shape
    out = np.empty(n, dtype=np.int32)
    for r0 in range(0, n, block_rows):
        rows = stored_draft[r0:r0 + block_rows]
        z = (bf16_to_f32(rows) if dtype == "bf16" else rows).astype(np.float64)
        g = -np.log(-np.log(rng.random(z.shape)))
        out[r0:r0 + block_rows] = np.argmax(z / temperature + g, axis=1)
    return out


def _argmax_tokens(stored_draft: np.ndarray, dtype: str) -> np.ndarray:
    z = bf16_to_f32(stored_draft) if dtype == "bf16" else stored_draft
    return np.argmax(z, axis=1).astype(np.int32)  # first occurrence on ties


def make_random(name: str, depths, V: int, dtype: str, temperature: float, target_sigma: float,
                draft_sigma, data_seed: int, verify_seed: int, greedy_drafts: bool | None = None,
                keep_draft: bool | None = None) -> Batch:
    """Gaussian-logit batch with the given per-request depths.

    draft_sigma: scalar or one value per request (noise added to the target logits).
    At temperature 0 the drafter proposes its argmax and the draft logits are not kept unless asked.
    """
    rng = np.random.Generator(np.random.Philox(data_seed))
    depths = np.asarray(depths, dtype=np.int64)
    B = depths.shape[0]
    cu = offsets_from_depths(depths)
    n_d = int(cu[-1])
    sig = np.broadcast_to(np.asarray(draft_sigma, dtype=np.float64), (B,))
    tgt = rng.standard_normal((n_d + B, V), dtype=np.float32)
    tgt *= np.float32(target_sigma)
    # draft row (i, j) perturbs target row (i, j)
    t_of_d = np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(B)]).astype(np.int64)
    req_of_d = np.repeat(np.arange(B), depths)
    drf = rng.standard_normal((n_d, V), dtype=np.float32)
    drf *= sig[req_of_d].astype(np.float32)[:, None]
    drf += tgt[t_of_d]
    target = _store(tgt, dtype)
    del tgt
    draft = _store(drf, dtype)
    del drf
    greedy = temperature == 0 if greedy_drafts is None else greedy_drafts
    tokens = _argmax_tokens(draft, dtype) if greedy else _gumbel_tokens(rng, draft, dtype, temperature)
    if keep_draft is None:
        keep_draft = temperature > 0
    return Batch(name=name, V=V, dtype=dtype, temperature=float(temperature), seed=int(verify_seed),
                 target=target, draft=draft if keep_draft else None, tokens=tokens, cu=cu,
                 meta={"data_seed": data_seed, "target_sigma": target_sigma,
                       "draft_sigma": np.asarray(draft_sigma).tolist()})


def with_profiles(b: Batch, temps, seeds, token_seed: int) -> Batch:
    """The same logits under one sampling profile per request: each request's draft tokens are
    redrawn from its own draft rows at its own temperature (the argmax where T_i = 0)."""
    if b.draft is None:
        raise ValueError("profiles need the draft logits")
    temps = np.asarray(temps, dtype=np.float32).reshape(b.B)
    seeds = np.asarray(seeds, dtype=np.uint64).reshape(b.B)
    rng = np.random.Generator(np.random.Philox(token_seed))
    req_of_d = np.repeat(np.arange(b.B), b.depths)
    tokens = _argmax_tokens(b.draft, b.dtype)
    sampled = np.nonzero(temps[req_of_d] > 0)[0]
    for r0 in range(0, sampled.size, 64):
        rows = sampled[r0:r0 + 64]
        z = (bf16_to_f32(b.draft[rows]) if b.dtype == "bf16" else b.draft[rows]).astype(np.float64)
        g = -np.log(-np.log(rng.random(z.shape)))
        tokens[rows] = np.argmax(z / temps[req_of_d[rows]].astype(np.float64)[:, None] + g, axis=1)
    return Batch(name=b.name + "_profiled", V=b.V, dtype=b.dtype, temperature=float("nan"), seed=0,
                 target=b.target, draft=b.draft, tokens=tokens.astype(np.int32), cu=b.cu,
                 meta=dict(b.meta, token_seed=token_seed), temp_each=temps, seed_each=seeds)


def with_qrows(b: Batch, temperature: float | None = None) -> Batch:
    """The same batch with the draft side given as distributions (SDCP's q_rows): each row is
    softmax(stored draft logits / T) in float64, rounded to float32; the draft tokens stay as drawn
    from the draft logits at T (the same distribution)."""
    if b.draft is None:
        raise ValueError("q rows are built from the draft logits")
    T = b.temperature if temperature is None else temperature
    q = np.empty((b.n_draft_rows, b.V), dtype=np.float32)
    for r0 in range(0, b.n_draft_rows, 64):
        z = (bf16_to_f32(b.draft[r0:r0 + 64]) if b.dtype == "bf16" else b.draft[r0:r0 + 64]).astype(np.float64) / T
        z -= z.max(axis=1, keepdims=True)
        e = np.exp(z)
        q[r0:r0 + 64] = e / e.sum(axis=1, keepdims=True)
    return Batch(name=b.name + "_qrows", V=b.V, dtype=b.dtype, temperature=b.temperature, seed=b.seed,
                 target=b.target, draft=None, tokens=b.tokens, cu=b.cu, meta=dict(b.meta),
                 temp_each=b.temp_each, seed_each=b.seed_each, qrows=q)


def with_truncation(b: Batch, top_k: int, top_p_milli: int) -> Batch:
    """The same logits under a truncating profile (top-k, then top-p, after the temperature) on
    every request.  The drafter proposes its argmax, the first rank of its row, which every
    truncation keeps, so every proposal is valid without the generator computing a kept set."""
    if b.draft is None:
        raise ValueError("a truncated batch needs the draft logits")
    return Batch(name=f"{b.name}_topk{top_k}_topp{top_p_milli}", V=b.V, dtype=b.dtype, temperature=b.temperature,
                 seed=b.seed, target=b.target, draft=b.draft, tokens=_argmax_tokens(b.draft, b.dtype), cu=b.cu,
                 meta=dict(b.meta, drafts="argmax"), temp_each=b.temp_each, seed_each=b.seed_each,
                 top_k=np.full(b.B, top_k, dtype=np.int32), top_p_milli=np.full(b.B, top_p_milli, dtype=np.int32))


def mixed_profiles(B: int, rng: np.random.Generator, temps=(0.0, 0.6, 1.0, 1.5)) -> tuple[np.ndarray, np.ndarray]:
    """Temperatures drawn from ``temps`` and distinct 64-bit seeds, one per request."""
    t = np.asarray(temps, dtype=np.float32)[rng.integers(0, len(temps), size=B)]
    seeds = rng.integers(0, 2**63, size=B, dtype=np.int64).astype(np.uint64) * np.uint64(2) + np.uint64(1)
    return t, seeds


# ----------------------------------------------------------------------------- the five workloads

DATA_SEED_BASE = 20261202


def small_b1(round_index: int = 0) -> Batch:
    """B=1, K=4, V=1000, fp32: target ~ N(0, 2^2), draft = target + N(0, 1), T = 1; one of 100 rounds."""
    return make_random("b1_k4_v1000_fp32", [4], 1000, "fp32", 1.0, 2.0, 1.0,
                       data_seed=DATA_SEED_BASE + 1000 + round_index, verify_seed=1000 + round_index)


def exactness_case(case: int, B: int = 4096, K: int = 3, V: int = 8):
    """One fixed (target, draft) row pair per case, reused at every position of every request.

    target ~ N(0, 1.5^2), draft = target + N(0, 0.7^2), fp32, T = 1.  Returns the two rows; batches
    with fresh draft tokens per trial come from ``exactness_batch``.
    """
    rng = np.random.Generator(np.random.Philox(DATA_SEED_BASE + 2000 + case))
    zt = (rng.standard_normal(V) * 1.5).astype(np.float32)
    zd = (zt + rng.standard_normal(V) * 0.7).astype(np.float32)
    return zt, zd


def exactness_batch(case: int, trial_block: int, B: int = 4096, K: int = 3, V: int = 8,
                    rows: tuple[np.ndarray, np.ndarray] | None = None) -> Batch:
    """B requests of depth K sharing one row pair; the draft tokens are redrawn per trial block."""
    zt, zd = exactness_case(case, B, K, V) if rows is None else rows
    cu = offsets_from_depths(np.full(B, K))
    target = np.ascontiguousarray(np.broadcast_to(zt, (B * (K + 1), V)), dtype=np.float32)
    draft = np.ascontiguousarray(np.broadcast_to(zd, (B * K, V)), dtype=np.float32)
    rng = np.random.Generator(np.random.Philox([DATA_SEED_BASE + 2000 + case, trial_block + 1]))
    g = -np.log(-np.log(rng.random((B * K, V))))
    tokens = np.argmax(zd.astype(np.float64)[None, :] + g, axis=1).astype(np.int32)
    return Batch(name="exact_b4096_k3_v8_fp32", V=V, dtype="fp32", temperature=1.0,
                 seed=(case << 32) | trial_block, target=target, draft=draft, tokens=tokens, cu=cu,
                 meta={"case": case, "trial_block": trial_block})


def small_b1_v128256(data_seed: int = DATA_SEED_BASE + 8, verify_seed: int = 8000) -> Batch:
    """B=1, K=4, V=128256, bf16: target ~ N(0, 3^2), draft = target + N(0, 1.5^2), T = 1 (one request
    of the target workload's vocabulary: the latency of a lone session's round)."""
    return make_random("b1_k4_v128256_bf16", [4], 128256, "bf16", 1.0, 3.0, 1.5, data_seed=data_seed,
                       verify_seed=verify_seed)


def uniform_b64(data_seed: int = DATA_SEED_BASE + 3, verify_seed: int = 3000) -> Batch:
    """B=64, K=5, V=32000, bf16: target ~ N(0, 3^2), draft = target + N(0, 1.5^2), T = 0.8."""
    return make_random("b64_k5_v32000_bf16", np.full(64, 5), 32000, "bf16", 0.8, 3.0, 1.5,
                       data_seed=data_seed, verify_seed=verify_seed)


def ragged_b256(data_seed: int = DATA_SEED_BASE + 4, verify_seed: int = 4000, B: int = 256,
                V: int = 128256) -> Batch:
    """B=256, K_i ~ U{0..8}, V=128256, bf16: target ~ N(0, 3^2), draft = target + N(0, s_i^2) with
    s_i ~ U[0.5, 3] per request, T = 1."""
    rng = np.random.Generator(np.random.Philox([data_seed, 7]))
    depths = rng.integers(0, 9, size=B)
    sig = rng.uniform(0.5, 3.0, size=B)
    return make_random(f"b{B}_ragged_k0to8_v{V}_bf16", depths, V, "bf16", 1.0, 3.0, sig,
                       data_seed=data_seed, verify_seed=verify_seed)


def greedy_b512(data_seed: int = DATA_SEED_BASE + 5, verify_seed: int = 5000, B: int = 512,
                V: int = 151936) -> Batch:
    """B=512, K=4, V=151936, bf16, T=0: target ~ N(0, 4^2), draft = target + N(0, 1); the drafter
    proposes its argmax; ties go to the lowest index."""
    return make_random(f"greedy_b{B}_k4_v{V}_bf16", np.full(B, 4), V, "bf16", 0.0, 4.0, 1.0,
                       data_seed=data_seed, verify_seed=verify_seed)


def tree_parents(kind: str, n: int, rng: np.random.Generator, branching: int = 2) -> np.ndarray:
    """Parents of an n-node tree in node order (every parent precedes its children; -1 is the
    root): "chain", "star" (all children of the root), "kary" (breadth-first, `branching` children
    per node), or "random" (each node's parent uniform over the root and the earlier nodes)."""
    if kind == "chain":
        return np.arange(-1, n - 1, dtype=np.int32)
    if kind == "star":
        return np.full(n, -1, dtype=np.int32)
    if kind == "kary":
        return np.array([(k // branching) - 1 if k >= branching else -1 for k in range(n)], dtype=np.int32)
    if kind == "random":
        return np.array([rng.integers(-1, k) if k > 0 else -1 for k in range(n)], dtype=np.int32)
    raise ValueError(kind)


def make_tree(name: str, sizes, kind: str, V: int, dtype: str, temperature: float, target_sigma: float,
              draft_sigma: float, data_seed: int, verify_seed: int, branching: int = 2, shared: bool = False) -> Batch:
    """Token-tree batch: request i holds sizes[i] nodes in the given shape.  Target rows are
    Gaussian (row 0 of a request at the root, row n + 1 after node n).  The drafter's row at a node's
    context is that context's target row plus Gaussian noise, shared by all of the node's children
    (draft row of node n = the row its token was drawn from), and each child's token is drawn from
    it independently (Gumbel-max at temperature T, or its argmax at T = 0).  shared: the draft side
    holds that row once per parent context, and draft_row gives each node's row (else one copy per
    node)."""
    rng = np.random.Generator(np.random.Philox(data_seed))
    sizes = np.asarray(sizes, dtype=np.int64)
    B = sizes.shape[0]
    cu = offsets_from_depths(sizes)
    n = int(cu[-1])
    parents = np.concatenate([tree_parents(kind, int(k), rng, branching) for k in sizes]).astype(np.int32) \
        if n else np.zeros(0, dtype=np.int32)
    tgt = rng.standard_normal((n + B, V), dtype=np.float32)
    tgt *= np.float32(target_sigma)
    noise = rng.standard_normal((n + B, V), dtype=np.float32)  # one drafter row per context (target row)
    noise *= np.float32(draft_sigma)
    req = np.repeat(np.arange(B), sizes)
    ctx_row = cu[req] + req + parents + 1  # the target row of each node's parent context
    drf = tgt[ctx_row] + noise[ctx_row]
    target = _store(tgt, dtype)
    draft = _store(drf, dtype)
    del tgt, noise, drf
    tokens = _argmax_tokens(draft, dtype) if temperature == 0 else _gumbel_tokens(rng, draft, dtype, temperature)
    draft_row = None
    if shared:  # one row per parent context, in context order
        ctx, first, draft_row = np.unique(ctx_row, return_index=True, return_inverse=True)
        draft = np.ascontiguousarray(draft[first])
        draft_row = draft_row.astype(np.int32)
    return Batch(name=name, V=V, dtype=dtype, temperature=float(temperature), seed=int(verify_seed),
                 target=target, draft=draft if temperature > 0 else None, tokens=tokens, cu=cu, parents=parents,
                 draft_row=draft_row,
                 meta={"data_seed": data_seed, "kind": kind, "target_sigma": target_sigma, "draft_sigma": draft_sigma})
