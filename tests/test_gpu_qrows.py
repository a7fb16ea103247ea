"""GPU parity of probability-row draft input (SDCP's q_rows, sdv_options.draft_probs) against the
fp64 oracle given the same rows: verdicts bit for bit up to counted near-ties, p/q ratios to 1e-5
relative; a zero q at a proposed token rejects that request alone."""
import numpy as np
import pytest
import torch

import workloads as W
import lossless_draft_verification_online_amd as sdv
from gpu_helpers import DEV, check_parity, log, run_gpu, run_oracle, to_device_off_grid
from oracle.compare import compare_verdicts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("V,dtype,T", [(32000, "bf16", 1.0), (20011, "bf16", 0.8), (8192, "bf16", 1.2), (8195, "bf16", 1.0),
                                       (4096, "fp32", 1.0), (1001, "fp32", 0.7), (13, "fp32", 1.0)])
def test_qrows_match_oracle(V, dtype, T):
    rng = np.random.default_rng(V)
    b = W.with_qrows(W.make_random(f"q_v{V}", rng.integers(0, 9, size=40), V, dtype, T, 3.0, 1.5, data_seed=V,
                                   verify_seed=5))
    acc, out, ref, cmp, dg = check_parity(b, diag=("ratio", "target_lse", "terminal_kind"))
    np.testing.assert_allclose(dg["ratio"], ref["ratio"], rtol=1e-5)
    np.testing.assert_allclose(np.exp(dg["target_lse"] - ref["target_lse"]), 1.0, rtol=1e-5)
    log(f"  {cmp['n_excused']} near-tie excuses, {(ref['terminal_kind'] == 2).sum()} corrections")


@pytest.mark.parametrize("V,dtype,tshift,qshift", [(4096, "fp32", 0, 1), (8192, "bf16", 0, 3), (8192, "bf16", 5, 2),
                                                   (20011, "bf16", 3, 1), (1003, "fp32", 2, 0)])
def test_qrows_off_the_16_byte_grid(V, dtype, tshift, qshift):
    """Target logits and q rows at bases off the 16-byte grid (shifted by whole elements): the pass
    splits each pair on the q row's grid and cuts the target logits under every q vector from two
    aligned pieces; verdicts against the oracle on the same rows."""
    rng = np.random.default_rng(V + 10 * tshift + qshift)
    b = W.with_qrows(W.make_random(f"q_off_v{V}_{tshift}_{qshift}", rng.integers(0, 9, size=32), V, dtype, 1.0, 3.0,
                                   1.5, data_seed=V + 7, verify_seed=9))
    log(f"  q rows off the grid: V={V} {dtype} target shift {tshift}, q shift {qshift}")
    t = to_device_off_grid(b.target, dtype, tshift)
    q = to_device_off_grid(b.qrows, "fp32", qshift)
    acc, out, dg = sdv.verify_ex(t, None, torch.from_numpy(b.tokens).to(DEV), torch.from_numpy(b.cu).to(DEV),
                                 b.temperature, b.seed, draft_probs=q, diag=("terminal_kind",))
    torch.cuda.synchronize()
    ref = run_oracle(b)
    cmp = compare_verdicts(acc.cpu().numpy(), out.cpu().numpy(), ref, b.cu, b.temperature)
    assert cmp["n_hard"] == 0, cmp["hard"][:10]
    assert (dg["terminal_kind"].cpu().numpy() == 2).any()  # corrections ran through the split pass


def test_full_size_ragged_b256_qrows():
    check_parity(W.with_qrows(W.ragged_b256()))


def test_qrows_with_profiles():
    rng = np.random.default_rng(3)
    base = W.make_random("q_prof", rng.integers(0, 9, size=64), 20011, "bf16", 1.0, 3.0, 1.0, data_seed=3,
                         verify_seed=0, keep_draft=True)
    t, s = W.mixed_profiles(base.B, rng, temps=(0.0, 0.9, 1.3))
    pb = W.with_profiles(base, t, s, token_seed=4)
    # each request's q rows at its own temperature (greedy requests: any rows, never read)
    q = np.empty((pb.n_draft_rows, pb.V), dtype=np.float32)
    req = np.repeat(np.arange(pb.B), pb.depths)
    for T in np.unique(t):
        rows = np.nonzero(t[req] == T)[0]
        if rows.size:
            sub = W.Batch(name="x", V=pb.V, dtype=pb.dtype, temperature=float(T) if T > 0 else 1.0, seed=0,
                          target=pb.target, draft=pb.draft[rows], tokens=pb.tokens[rows],
                          cu=W.offsets_from_depths([rows.size]))
            q[rows] = W.with_qrows(sub).qrows
    pb.qrows = q
    pb.draft = None
    check_parity(pb)


def test_zero_q_at_the_token_rejects_only_that_request():
    b = W.with_qrows(W.make_random("q_zero", [3, 4, 2], 4096, "fp32", 1.0, 2.0, 1.0, data_seed=8, verify_seed=2))
    d = b.cu[1] + 2
    b.qrows[d, b.tokens[d]] = 0.0
    acc, out, dg = run_gpu(b, diag=("terminal_kind",))
    assert acc[1] == -1 and dg["terminal_kind"][1] == -1 and (out[b.cu[1] + 1: b.cu[2] + 2] == -1).all()
    ref = run_oracle(b)
    assert ref["accepted_len"][1] == -1
    for i in (0, 2):
        s = slice(b.cu[i] + i, b.cu[i + 1] + i + 1)
        assert acc[i] == ref["accepted_len"][i] and np.array_equal(out[s], ref["out_tokens"][s])


@pytest.mark.parametrize("V,dtype", [(4096, "fp32"), (32000, "bf16"), (128256, "bf16")])
def test_empty_residual_falls_back_to_p(V, dtype):
    """q rows given as 1.5 p (used as given, SDCP's q_rows): every ratio is 2/3, and after a rejection
    max(p - q, 0) is zero at every token, so the extra token is drawn from p itself
    (SDV_TERM_RESIDUAL_EMPTY) on rows of 1, 4 and 16 chunks.  With logit drafts an empty residual
    cannot follow a rejection: it needs p <= q at every token, i.e. p = q, whose ratio 1 always
    accepts."""
    rng = np.random.default_rng(V + 1)
    b = W.with_qrows(W.make_random(f"q_empty_v{V}", rng.integers(1, 9, size=40), V, dtype, 1.0, 2.0, 1.0,
                                   data_seed=V + 2, verify_seed=6))
    z = b.target_f32().astype(np.float64)
    req = np.repeat(np.arange(b.B), b.depths)
    rows = b.cu[req] + req + (np.arange(b.n_draft_rows) - b.cu[req])  # the target row of each draft position
    p = np.exp(z[rows] - z[rows].max(axis=1, keepdims=True))
    b.qrows = (1.5 * p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    acc, out, ref, cmp, dg = check_parity(b, diag=("terminal_kind",))
    empty = ref["terminal_kind"] == 3
    assert empty.sum() >= 5, "the batch must exercise the empty residual"
    same = acc == ref["accepted_len"]
    assert np.array_equal(dg["terminal_kind"][same], ref["terminal_kind"][same])
