"""The seeded workload generator: shapes, determinism, ragged layout and bf16 encoding."""
import numpy as np

import workloads as W


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 65504.0], dtype=np.float32)
    bits = W.bf16_bits(x)
    back = W.bf16_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins; 1 + 3*2^-8 rounds up to 1 + 2^-6
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.015625)
    assert back[3] == -2.5
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0**-8)


def test_ragged_layout_and_determinism():
    a = W.make_random("t", [0, 3, 1, 0, 2], 64, "bf16", 1.0, 3.0, [0.5, 1, 2, 3, 1], 11, 22)
    b = W.make_random("t", [0, 3, 1, 0, 2], 64, "bf16", 1.0, 3.0, [0.5, 1, 2, 3, 1], 11, 22)
    assert a.cu.tolist() == [0, 0, 3, 4, 4, 6]
    assert a.target.shape == (6 + 5, 64) and a.draft.shape == (6, 64) and a.tokens.shape == (6,)
    assert np.array_equal(a.target, b.target) and np.array_equal(a.tokens, b.tokens)
    assert a.target.dtype == np.uint16 and a.tokens.dtype == np.int32
    assert ((a.tokens >= 0) & (a.tokens < 64)).all()
    assert a.algorithmic_bytes() == (11 + 6) * 64 * 2


def test_greedy_workload_drafts_argmax_and_drops_draft_logits():
    g = W.make_random("g", [4, 4], 100, "bf16", 0.0, 4.0, 1.0, 5, 6, keep_draft=True)
    z = W.bf16_to_f32(g.draft)
    assert np.array_equal(g.tokens, np.argmax(z, axis=1))
    g2 = W.make_random("g", [4, 4], 100, "bf16", 0.0, 4.0, 1.0, 5, 6)
    assert g2.draft is None and np.array_equal(g2.tokens, g.tokens)
    assert g2.algorithmic_bytes() == 10 * 100 * 2


def test_gumbel_draft_tokens_follow_draft_softmax():
    # the drafter samples x ~ softmax(z_d / T): check the empirical law on one fixed row
    rng = np.random.default_rng(0)
    zd = (rng.standard_normal(6) * 1.5).astype(np.float32)
    rows = np.tile(zd, (200000, 1))
    toks = W._gumbel_tokens(np.random.default_rng(1), rows, "fp32", 0.8)
    emp = np.bincount(toks, minlength=6) / toks.size
    ref = np.exp(zd / 0.8 - np.max(zd / 0.8))
    ref /= ref.sum()
    assert np.abs(emp - ref).max() < 5 * np.sqrt(ref.max() / toks.size)


def test_exactness_batch_shapes():
    b = W.exactness_batch(2, 0)
    assert b.B == 4096 and b.V == 8 and b.target.shape == (4096 * 4, 8) and b.draft.shape == (4096 * 3, 8)
    assert (b.target == b.target[0]).all() and (b.draft == b.draft[0]).all()
