"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded inputs.

Verdicts (accepted lengths and every emitted token id) must match the oracle bit for bit; the only
excuse is a first divergence at a decision the oracle took within 1e-6 of its threshold (|r - p/q|
or the CDF margin of the draw), counted by the comparator.  Greedy verdicts allow no excuse.
Intermediate values are checked too: log-normalisers and p/q ratios to 1e-5 relative on
probabilities, argmaxes exactly.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, check_parity, log, run_gpu, run_oracle, to_device, to_device_off_grid

pytestmark = pytest.mark.gpu

RTOL_PROB = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ----------------------------------------------------------------------------- Philox

def test_device_philox_matches_oracle():
    import lossless_draft_verification_online_amd as sdv
    from oracle import oracle
    rng = np.random.default_rng(0)
    n = 4096
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    ctr[:64] = 0
    key[:32] = 0
    out = sdv.philox4x32_10(torch.from_numpy(ctr.view(np.int32)).to(DEV),
                            torch.from_numpy(key.view(np.int32)).to(DEV)).cpu().numpy().view(np.uint32)
    for b in range(n):
        assert np.array_equal(out[b], oracle.philox4x32_10(ctr[b], key[b])), b


def test_device_uniforms_match_oracle_blocks():
    from oracle import oracle
    b = W.make_random("philox_layout", np.full(16, 8), 64, "fp32", 1.0, 1.0, 1.0, 3, 0xFEEDFACECAFEBEEF)
    _, _, dg = run_gpu(b, diag=("accept_uniform", "draw_uniform", "terminal_kind"))
    grid = oracle.philox_grid(b.seed, 16, 9)
    r = ((grid[:, :8, 0] >> 8) + 1).astype(np.float64) / 2**24
    assert np.array_equal(dg["accept_uniform"].astype(np.float64), r.reshape(-1))


# ----------------------------------------------------------------------------- row quantities

@pytest.mark.parametrize("V,dtype", [(1000, "fp32"), (32000, "bf16"), (8192, "bf16"), (8193, "bf16"),
                                     (20011, "bf16"), (13, "fp32"), (4099, "fp32"), (151936, "bf16"),
                                     (200003, "bf16")])
def test_row_lse_and_ratio(V, dtype):
    rng = np.random.default_rng(V)
    depths = rng.integers(0, 9, size=12)
    b = W.make_random(f"rows_v{V}", depths, V, dtype, 0.8, 3.0, rng.uniform(0.5, 3, 12), V, 77)
    _, _, dg = run_gpu(b, diag=("target_lse", "draft_lse", "ratio"))
    ref = run_oracle(b)
    # an LSE error dL is a relative probability error of about dL
    np.testing.assert_allclose(dg["target_lse"], ref["target_lse"], rtol=0, atol=RTOL_PROB)
    np.testing.assert_allclose(dg["draft_lse"], ref["draft_lse"], rtol=0, atol=RTOL_PROB)
    np.testing.assert_allclose(dg["ratio"], ref["ratio"], rtol=RTOL_PROB, atol=0)


@pytest.mark.parametrize("V", [1, 7, 8192, 8193, 151936])
def test_row_argmax_exact_with_ties(V):
    rng = np.random.default_rng(V + 5)
    depths = rng.integers(0, 5, size=16)
    b = W.make_random(f"argmax_v{V}", depths, V, "bf16", 0.0, 4.0, 1.0, V + 1, 0)
    # plant ties at the row maximum in half of the rows
    tv = W.bf16_to_f32(b.target).copy()
    for r in range(0, tv.shape[0], 2):
        k = min(V, 4)
        idx = rng.choice(V, size=k, replace=False)
        tv[r, idx] = tv[r].max() + 1.0
    b.target = W.bf16_bits(tv)
    _, _, dg = run_gpu(b, diag=("target_argmax",))
    np.testing.assert_array_equal(dg["target_argmax"], np.argmax(W.bf16_to_f32(b.target), axis=1))


@pytest.mark.parametrize("V,dtype,T,shift", [(8192, "bf16", 1.0, 3), (8192, "bf16", 0.0, 5), (4096, "fp32", 0.8, 1),
                                             (20011, "bf16", 1.0, 7), (20011, "bf16", 0.0, 1), (4099, "fp32", 0.0, 2),
                                             (9, "bf16", 0.0, 3)])
def test_rows_off_the_16_byte_grid(V, dtype, T, shift):
    """Logit bases on an element boundary only, so every chunk is read as head elements, 16-byte
    vectors and tail elements: normalisers, argmaxes and verdicts against the oracle, with maxima
    planted at a row's first and last element and ties between those edges and the vectors."""
    rng = np.random.default_rng(V + shift)
    depths = rng.integers(0, 7, size=12)
    b = W.make_random(f"offgrid_v{V}_{dtype}_s{shift}", depths, V, dtype, T, 3.0, rng.uniform(0.5, 3, 12), V + shift,
                      91)
    f32 = (lambda a: W.bf16_to_f32(a).copy()) if dtype == "bf16" else (lambda a: a.copy())
    back = W.bf16_bits if dtype == "bf16" else (lambda a: a.astype(np.float32))
    tv = f32(b.target)
    for r in range(tv.shape[0]):
        top = tv[r].max() + 1.0
        kind = r % 4
        if kind == 0:
            tv[r, 0] = top                      # the head's first element
        elif kind == 1:
            tv[r, V - 1] = top                  # the tail's last element
        elif kind == 2:
            tv[r, [0, V // 2]] = top            # a head element tied with a vector element
        else:
            tv[r, [V // 2, V - 1]] = top        # a vector element tied with a tail element
    b.target = back(tv)
    dev = (to_device_off_grid(b.target, dtype, shift), to_device_off_grid(b.draft, dtype, shift), torch.from_numpy(b.tokens).to(DEV),
           torch.from_numpy(b.cu).to(DEV))
    diag = ("target_argmax",) if T == 0.0 else ("target_lse", "draft_lse", "terminal_kind")
    _, _, ref, _, dg = check_parity(b, dev_inputs=dev, diag=diag)
    if T == 0.0:
        np.testing.assert_array_equal(dg["target_argmax"], np.argmax(tv, axis=1))
    else:
        np.testing.assert_allclose(dg["target_lse"], ref["target_lse"], rtol=0, atol=RTOL_PROB)
        np.testing.assert_allclose(dg["draft_lse"], ref["draft_lse"], rtol=0, atol=RTOL_PROB)


# ----------------------------------------------------------------------------- the five workloads

def test_workload_b1_v1000_fp32_100_rounds():
    n_exc = 0
    for rnd in range(100):
        _, _, _, cmp, _ = check_parity(W.small_b1(rnd))
        n_exc += cmp["n_excused"]
    log(f"  100 rounds: {n_exc} near-tie excuses")


def test_workload_exactness_v8_subset():
    for case in range(8):
        for blk in range(2):
            check_parity(W.exactness_batch(case, blk))


def test_workload_b64_v32000_bf16():
    for seed in range(4):
        check_parity(W.uniform_b64(verify_seed=3000 + seed))


def test_workload_b256_ragged_v128256_bf16_full():
    b = W.ragged_b256()
    dev_inputs = (to_device(b.target, b.dtype), to_device(b.draft, b.dtype), torch.from_numpy(b.tokens).to(DEV),
                  torch.from_numpy(b.cu).to(DEV))
    for seed in (4000, 4001):
        acc, out, ref, cmp, dg = check_parity(b, seed=seed, dev_inputs=dev_inputs)
        kinds = dg["terminal_kind"]
        log(f"  seed {seed}: mean accepted {acc.mean():.3f}, residual draws {(kinds == 2).sum()}, "
            f"bonus {(kinds == 1).sum()}, excused {cmp['n_excused']}")


def test_workload_greedy_b512_v151936_bf16_full():
    b = W.greedy_b512()
    acc, out, ref, cmp, dg = check_parity(b)
    assert cmp["n_excused"] == 0
    log(f"  greedy mean accepted {acc.mean():.3f}")


# ----------------------------------------------------------------------------- edge cases

def test_all_requests_k0():
    b = W.make_random("k0", np.zeros(37, int), 5000, "bf16", 1.0, 3.0, 1.0, 9, 10)
    acc, out, *_ = check_parity(b)
    assert (acc == 0).all()


def test_depth_64_and_mixed():
    b = W.make_random("k64", [64, 0, 63, 1, 64], 700, "fp32", 1.0, 1.0, 0.05, 10, 11)
    check_parity(b)
    g = W.make_random("k64g", [64, 0, 63, 1, 64], 700, "fp32", 0.0, 1.0, 0.0, 10, 11)
    acc, out, ref, cmp, _ = check_parity(g)
    assert acc[0] == 64 and acc[4] == 64  # the drafter proposes the target argmax itself


@pytest.mark.parametrize("V,dtype", [(1, "fp32"), (1, "bf16"), (7, "bf16"), (13, "fp32"), (8192, "bf16"),
                                     (8193, "bf16"), (65541, "bf16"), (4096, "fp32"), (4097, "fp32")])
def test_vocab_sizes_and_ragged_tails(V, dtype):
    rng = np.random.default_rng(V * 3 + len(dtype))
    depths = rng.integers(0, 9, size=20)
    for T in (1.0, 0.0):
        b = W.make_random(f"v{V}", depths, V, dtype, T, 2.0, rng.uniform(0.3, 2.0, 20), V + 3, 7)
        check_parity(b)


@pytest.mark.parametrize("V,dtype,t_from,d_from", [(20000, "bf16", 12000, 15000), (5000, "fp32", 4096, 4500),
                                                   (20003, "bf16", 16384, 16000)])
def test_masked_vocabulary(V, dtype, t_from, d_from):
    """Padded vocabularies: every target logit from t_from on and every draft logit from d_from on
    is -inf (whole chunks among them), so p and q vanish there, and the draft tokens are drawn from
    the masked draft rows.  Sampling (logit and probability draft rows) and greedy."""
    rng = np.random.default_rng(V + t_from)
    depths = rng.integers(0, 9, size=24)
    neg = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    for T in (1.0, 0.0):
        b = W.make_random(f"masked_v{V}", depths, V, dtype, T, 3.0, 1.5, V + 5, 19, keep_draft=True)
        b.target = b.target.copy()
        b.target[:, t_from:] = neg
        b.draft = b.draft.copy()
        b.draft[:, d_from:] = neg
        tok_rng = np.random.Generator(np.random.Philox(V + 23))
        b.tokens = W._gumbel_tokens(tok_rng, b.draft, dtype, T) if T > 0 else W._argmax_tokens(b.draft, dtype)
        assert (b.tokens < d_from).all()
        acc, *_ = check_parity(b)
        assert (acc >= 0).all()
        if T > 0:
            check_parity(W.with_qrows(b))


@pytest.mark.parametrize("T", [0.02, 0.1, 8.0, 50.0])
def test_extreme_temperatures(T):
    """Temperatures far from 1: nearly one-hot p and q (most exponentials underflow to 0, and the
    residual lives on a handful of tokens), and nearly flat ones (the ratio near 1 everywhere)."""
    rng = np.random.default_rng(int(T * 100) + 7)
    depths = rng.integers(0, 9, size=32)
    for V, dtype in ((32000, "bf16"), (3001, "fp32")):
        b = W.make_random(f"temp{T}_v{V}", depths, V, dtype, T, 3.0, rng.uniform(0.2, 2.0, 32), V + 9, 29)
        acc, *_ = check_parity(b)
        assert (acc >= 0).all()


@pytest.mark.parametrize("V,dtype,depths", [(1000, "fp32", [0, 1, 4, 7, 8]), (8192, "bf16", [0, 3, 7]),
                                            (16384, "bf16", [0, 1, 3, 4]), (24, "fp32", [5, 64])])
def test_one_request_batches(V, dtype, depths):
    """A batch of one request whose rows hold at most 16 chunks runs in a single launch (records,
    screening and verdict in one workgroup); deeper ones (K = 8 at one chunk per row, K = 4 at two,
    K = 64) take the two kernels.  Parity with the oracle at T > 0 and T = 0, one call per depth."""
    for K in depths:
        for T in (1.0, 0.0):
            b = W.make_random(f"one_v{V}_k{K}", [K], V, dtype, T, 3.0, 1.0, V + K, 41 + K)
            acc, *_ = check_parity(b)
            assert 0 <= acc[0] <= K


def test_one_request_with_bad_offsets_writes_nothing():
    """The single-launch path screens the offsets itself: cu[0] != 0 rejects the batch without
    writing a slot."""
    import lossless_draft_verification_online_amd as sdv
    b = W.make_random("one_bad", [3], 1000, "fp32", 1.0, 2.0, 1.0, 5, 6)
    t, d, x = to_device(b.target, "fp32"), to_device(b.draft, "fp32"), torch.from_numpy(b.tokens).to(DEV)
    cu = torch.tensor([1, 3], dtype=torch.int32, device=DEV)
    out = torch.full((b.n_draft_rows + 1,), -7, dtype=torch.int32, device=DEV)
    acc = torch.full((1,), 5, dtype=torch.int32, device=DEV)
    sdv.verify(t, d, x, cu, 1.0, 6, out=(acc, out))
    torch.cuda.synchronize()
    assert acc.cpu().tolist() == [-1]
    assert (out.cpu().numpy() == -7).all()


def test_bad_requests_are_isolated():
    rng = np.random.default_rng(21)
    depths = [3, 2, 4, 0, 5]
    b = W.make_random("bad", depths, 3000, "bf16", 1.0, 3.0, 1.0, 21, 22)
    good_acc, good_out, *_ = run_gpu(b)
    b.tokens = b.tokens.copy()
    b.tokens[b.cu[1] + 1] = 3000                     # request 1: token out of range
    d = W.bf16_to_f32(b.draft).copy()
    d[b.cu[2] + 3, b.tokens[b.cu[2] + 3]] = -np.inf  # request 2: q(x) = 0 at its last position
    b.draft = W.bf16_bits(d)
    acc, out, ref, cmp, _ = check_parity(b)
    assert acc[1] == -1 and acc[2] == -1
    assert (out[b.cu[1] + 1: b.cu[3] + 3] == -1).all()
    keep = [0, 3, 4]
    assert np.array_equal(acc[keep], good_acc[keep])


def test_depth_over_limit_writes_nothing():
    b = W.make_random("limit", [65, 2], 64, "fp32", 1.0, 1.0, 1.0, 5, 6)
    t, d, x, cu = (to_device(b.target, "fp32"), to_device(b.draft, "fp32"), torch.from_numpy(b.tokens).to(DEV),
                   torch.from_numpy(b.cu).to(DEV))
    import lossless_draft_verification_online_amd as sdv
    out = torch.full((b.n_draft_rows + 2,), -7, dtype=torch.int32, device=DEV)
    acc = torch.empty(2, dtype=torch.int32, device=DEV)
    sdv.verify(t, d, x, cu, 1.0, 6, out=(acc, out))
    torch.cuda.synchronize()
    assert acc.cpu().tolist()[0] == -1 and acc.cpu().tolist()[1] >= 0
    assert (out[:66].cpu().numpy() == -7).all()


def test_draft_equal_to_target_accepts_all():
    rng = np.random.default_rng(3)
    depths = rng.integers(0, 9, size=32)
    b = W.make_random("same", depths, 40000, "bf16", 1.0, 3.0, 0.0, 31, 32)
    acc, out, ref, cmp, dg = check_parity(b, diag=("ratio", "terminal_kind"))
    assert np.array_equal(acc, depths)
    assert (dg["ratio"] == 1.0).all()


def test_repeat_launches_are_deterministic():
    b = W.uniform_b64()
    ins = (to_device(b.target, b.dtype), to_device(b.draft, b.dtype), torch.from_numpy(b.tokens).to(DEV),
           torch.from_numpy(b.cu).to(DEV))
    first = run_gpu(b, dev_inputs=ins, diag=("target_lse", "ratio"))
    for _ in range(20):
        again = run_gpu(b, dev_inputs=ins, diag=("target_lse", "ratio"))
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])
        assert np.array_equal(first[2]["target_lse"], again[2]["target_lse"])
        assert np.array_equal(first[2]["ratio"], again[2]["ratio"], equal_nan=True)


# ----------------------------------------------------------------------------- read yardstick

def test_read_ceiling_folds_every_word():
    import lossless_draft_verification_online_amd as sdv
    rng = np.random.default_rng(11)
    n_chunks = 1037
    words = rng.integers(0, 2**32, size=n_chunks * 4096, dtype=np.uint64).astype(np.uint32)
    got = sdv.read_ceiling(torch.from_numpy(words.view(np.int32)).to(DEV)).cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(words.reshape(n_chunks, 4096), axis=1)
    assert np.array_equal(got, want)


# ----------------------------------------------------------------------------- size edges

@pytest.mark.parametrize("V,dtype", [(262144, "bf16"), (128255, "bf16"), (151936, "fp32")])
def test_large_and_odd_vocabularies(V, dtype):
    """32 chunks per row (4 per wave in the residual pass), an odd vocabulary on the element-wise
    path, and fp32 rows at the greedy workload's width."""
    rng = np.random.default_rng(V % 1000)
    b = W.make_random(f"v{V}_{dtype}", rng.integers(0, 9, size=24), V, dtype, 1.0, 3.0, rng.uniform(0.5, 3, 24),
                      data_seed=V, verify_seed=11)
    check_parity(b, diag=("terminal_kind", "target_lse"))


@pytest.mark.parametrize("V,dtype,B", [(12288, "fp32", 32), (24576, "bf16", 128), (16384, "bf16", 7)])
def test_small_batches_of_short_rows(V, dtype, B):
    """Batches of at most 128 requests on 16-byte rows of two to four chunks take the verdict kernel
    with 16 waves per request (the single pass over the rejected pair, the quarter-stage mass pass
    form); verdicts and normalisers against the oracle."""
    rng = np.random.default_rng(V + B)
    b = W.make_random(f"short_rows_v{V}_b{B}", rng.integers(0, 9, size=B), V, dtype, 0.9, 3.0,
                      rng.uniform(0.5, 3, B), data_seed=V + B, verify_seed=21)
    _, _, ref, cmp, dg = check_parity(b, diag=("terminal_kind", "target_lse"))
    np.testing.assert_allclose(dg["target_lse"], ref["target_lse"], rtol=0, atol=RTOL_PROB)
    assert (ref["terminal_kind"] == 2).any()


def test_one_request_at_full_depth_and_width():
    b = W.make_random("b1_k64_v128256", [64], 128256, "bf16", 1.0, 3.0, 0.3, data_seed=64, verify_seed=64)
    acc, out, ref, cmp, _ = check_parity(b)
    log(f"  accepted {acc[0]} of 64")


def test_every_request_without_drafts_at_full_width():
    b = W.make_random("b256_k0_v128256", np.zeros(256, dtype=int), 128256, "bf16", 1.0, 3.0, 1.0, data_seed=3,
                      verify_seed=3)
    acc, out, ref, cmp, dg = check_parity(b, diag=("terminal_kind",))
    assert (acc == 0).all() and (dg["terminal_kind"] == 1).all()
