"""GPU parity of per-request sampling profiles (sdv_verify_profiled) against the fp64 oracle.

Each request carries its own temperature and seed (SDCP "Session Contract"; a batch gathers many
sessions).  Verdicts must match the oracle's bit for bit up to counted near-ties, as for one
profile per batch; a batch whose profiles are all equal must reproduce the single-profile entry
point exactly; a temperature that describes no profile rejects its request alone.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, check_parity, log, profile_args, run_gpu, run_oracle, to_device
from oracle.compare import compare_verdicts

pytestmark = pytest.mark.gpu

RTOL_PROB = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _profiled(name, depths, V, dtype, seed, temps=(0.0, 0.6, 1.0, 1.5), draft_sigma=1.5):
    rng = np.random.default_rng(seed)
    b = W.make_random(name, depths, V, dtype, 1.0, 3.0, draft_sigma, data_seed=seed, verify_seed=0, keep_draft=True)
    t, s = W.mixed_profiles(b.B, rng, temps)
    return W.with_profiles(b, t, s, token_seed=seed + 1)


@pytest.mark.parametrize("V,dtype", [(32000, "bf16"), (20011, "bf16"), (1001, "fp32"), (4096, "fp32"), (8193, "bf16")])
def test_mixed_profiles_match_oracle(V, dtype):
    rng = np.random.default_rng(V)
    b = _profiled(f"mixed_v{V}", rng.integers(0, 9, size=48), V, dtype, seed=V)
    acc, out, ref, cmp, dg = check_parity(b, diag=("target_lse", "draft_lse", "ratio", "target_argmax", "terminal_kind"))
    log(f"  {cmp['n_excused']} near-tie excuses; temperatures {sorted(set(b.temp_each.tolist()))}")
    samp = b.temp_each > 0
    req_of_t = np.repeat(np.arange(b.B), b.depths + 1)
    req_of_d = np.repeat(np.arange(b.B), b.depths)
    # log-normalisers of sampling requests, probabilities to 1e-5 relative
    t_rows = samp[req_of_t]
    np.testing.assert_allclose(np.exp(dg["target_lse"][t_rows] - ref["target_lse"][t_rows]), 1.0, rtol=RTOL_PROB)
    d_rows = samp[req_of_d]
    np.testing.assert_allclose(np.exp(dg["draft_lse"][d_rows] - ref["draft_lse"][d_rows]), 1.0, rtol=RTOL_PROB)
    np.testing.assert_allclose(dg["ratio"][d_rows], ref["ratio"][d_rows], rtol=RTOL_PROB)
    # argmaxes of greedy requests exactly
    g_rows = ~samp[req_of_t]
    assert np.array_equal(dg["target_argmax"][g_rows], ref["target_argmax"][g_rows])
    assert np.array_equal(dg["terminal_kind"][~samp], np.zeros((~samp).sum()))


def test_full_size_ragged_b256_mixed_profiles():
    base = W.ragged_b256()
    rng = np.random.default_rng(44)
    t, s = W.mixed_profiles(base.B, rng)
    b = W.with_profiles(base, t, s, token_seed=45)
    check_parity(b)


def test_uniform_profile_equals_single_profile_entry_point():
    for T in (0.8, 0.0):
        b = W.make_random("same", np.random.default_rng(3).integers(0, 9, size=40), 20011, "bf16", 1.0, 3.0, 1.5,
                          data_seed=3, verify_seed=99, keep_draft=True)
        pb = W.with_profiles(b, np.full(b.B, T), np.full(b.B, 99), token_seed=4)
        ins = (to_device(pb.target, pb.dtype), to_device(pb.draft, pb.dtype), torch.from_numpy(pb.tokens).to(DEV),
               torch.from_numpy(pb.cu).to(DEV))
        prof = run_gpu(pb, dev_inputs=ins, diag=("target_lse", "ratio", "target_argmax"))
        # the profile carries T as binary32; the single-profile call gets the same value
        single = W.Batch(name="same", V=pb.V, dtype=pb.dtype, temperature=float(np.float32(T)), seed=99, target=pb.target,
                         draft=pb.draft, tokens=pb.tokens, cu=pb.cu)
        one = run_gpu(single, dev_inputs=ins, diag=("target_lse", "ratio", "target_argmax"))
        assert np.array_equal(prof[0], one[0]) and np.array_equal(prof[1], one[1]), T
        key = "target_argmax" if T == 0 else "target_lse"
        assert np.array_equal(prof[2][key], one[2][key], equal_nan=True), T


@pytest.mark.parametrize("bad_T", [-1.0, float("nan"), float("inf"), 1e-40])
def test_invalid_temperature_rejects_only_its_request(bad_T):
    b = _profiled("bad_profile", np.random.default_rng(9).integers(1, 9, size=24), 4099, "fp32", seed=9)
    temps = b.temp_each.copy()
    temps[6] = bad_T
    b.temp_each = temps
    acc, out, dg = run_gpu(b, diag=("terminal_kind",))
    lo, hi = b.cu[6] + 6, b.cu[7] + 7
    assert acc[6] == -1 and (out[lo:hi] == -1).all() and dg["terminal_kind"][6] == -1
    # every other request as the oracle has it (the oracle sees a harmless temperature there)
    temps_ok = temps.copy()
    temps_ok[6] = 1.0
    b.temp_each = temps_ok
    ref = run_oracle(b)
    cmp = compare_verdicts(acc, out, ref, b.cu, temps_ok.astype(np.float64))
    assert [i for i, _ in cmp["hard"]] == [6], cmp["hard"]


def test_profiled_host_argument_errors():
    import lossless_draft_verification_online_amd as sdv
    b = _profiled("args", [2, 3], 64, "fp32", seed=1)
    t, d, x, cu = to_device(b.target, "fp32"), to_device(b.draft, "fp32"), torch.from_numpy(b.tokens).to(DEV), \
        torch.from_numpy(b.cu).to(DEV)
    temp, seed = profile_args(b)
    with pytest.raises(ValueError):
        sdv.verify_ex(t, None, x, cu, temp, seed)  # draft rows exist, so the draft logits are needed
    with pytest.raises(ValueError):
        sdv.verify_ex(t, d, x, cu, temp, 5)  # both or neither as tensors
    with pytest.raises(ValueError):
        sdv.verify_ex(t, d, x, cu, temp[:1], seed[:1])
