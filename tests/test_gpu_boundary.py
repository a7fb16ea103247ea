"""GPU tests of the boundary itself: sdv_verify called straight through ctypes, the diagnostic
gathers and terminal mass of sdv_diag, the verifier's Philox blocks (sdv_philox_uniforms), and
requests too deep for the verdict kernel to stage their chunk records in shared memory.

Expected values come from the fp64 oracle or, for the gathers, from the stored inputs themselves.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, check_parity, log, run_gpu, run_oracle, upload
from lossless_draft_verification_online_amd import _native
from oracle import oracle
from oracle.compare import compare_verdicts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ptr(t):
    return None if t is None else t.data_ptr()


@pytest.mark.parametrize("dtype,V,T", [("bf16", 32000, 1.0), ("fp32", 1000, 0.8), ("bf16", 151936, 0.0)])
def test_sdv_verify_entry_point_against_oracle(dtype, V, T):
    """The benchmark spec's own entry point, sdv_verify, called through ctypes on a real batch."""
    rng = np.random.default_rng(V)
    depths = rng.integers(0, 9, size=24)
    b = W.make_random(f"sdv_verify_{dtype}_{V}", depths, V, dtype, T, 3.0, rng.uniform(0.5, 3.0, size=24),
                      data_seed=int(V) + 7, verify_seed=0xABCDEF0123 + V)
    log(f"  sdv_verify {b.name}: B={b.B} n_d={b.n_draft_rows} T={T}")
    t, d, x, cu = upload(b)
    lib = _native.lib()
    dt = _native.SDV_BF16 if dtype == "bf16" else _native.SDV_FP32
    need = lib.sdv_workspace_bytes(b.B, b.n_draft_rows, V, dt)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    acc = torch.full((b.B,), -9, dtype=torch.int32, device=DEV)
    out = torch.full((b.n_draft_rows + b.B,), -9, dtype=torch.int32, device=DEV)
    with torch.cuda.device(DEV):
        rc = lib.sdv_verify(_ptr(t), _ptr(d), _ptr(x), _ptr(cu), b.B, b.n_draft_rows, V, dt, T, b.seed,
                            _ptr(acc), _ptr(out), _ptr(ws), need, torch.cuda.current_stream(DEV).cuda_stream)
    assert rc == 0, lib.sdv_status_string(rc)
    torch.cuda.synchronize()
    ref = run_oracle(b)
    cmp = compare_verdicts(acc.cpu().numpy(), out.cpu().numpy(), ref, b.cu, T)
    assert cmp["n_hard"] == 0, cmp["hard"][:10]
    if T == 0.0:
        assert cmp["n_excused"] == 0


def _gathers_expected(b):
    tgt, drf = b.target_f32(), b.draft_f32()
    rows_t = np.concatenate([np.arange(b.cu[i], b.cu[i + 1]) + i for i in range(b.B)]).astype(int)
    return tgt[rows_t, b.tokens], drf[np.arange(b.n_draft_rows), b.tokens]


@pytest.mark.parametrize("case", ["bf16_32000", "fp32_1000_one_chunk", "fp32_4099_unaligned", "bf16_b1_split"])
def test_diag_gathers_and_terminal_mass(case):
    """z_t[x] and z_d[x] equal the stored logits at the draft tokens; the terminal mass S equals the
    oracle's total weight of the same draw (correction: sum of max(p - q, 0); bonus: mass of p)."""
    rng = np.random.default_rng(len(case))
    if case == "bf16_32000":
        b = W.make_random(case, rng.integers(0, 9, size=40), 32000, "bf16", 1.0, 3.0, rng.uniform(0.5, 3, 40), 11, 21)
    elif case == "fp32_1000_one_chunk":
        b = W.make_random(case, rng.integers(0, 6, size=64), 1000, "fp32", 1.0, 2.0, 1.0, 12, 22)
    elif case == "fp32_4099_unaligned":
        b = W.make_random(case, rng.integers(0, 6, size=32), 4099, "fp32", 0.9, 2.0, 1.5, 13, 23)
    else:  # one request: the correction's residual pass is shared among several workgroups
        b = W.make_random(case, [6], 128256, "bf16", 1.0, 3.0, 3.0, 14, 24)
    log(f"  diag {b.name}: B={b.B} V={b.V}")
    acc, out, dg = run_gpu(b, diag=("target_logit", "draft_logit", "terminal_mass", "terminal_kind"))
    ref = run_oracle(b)
    cmp = compare_verdicts(acc, out, ref, b.cu, b.temperature)
    assert cmp["n_hard"] == 0
    zt, zd = _gathers_expected(b)
    valid_d = np.repeat(acc >= 0, np.diff(b.cu))
    assert np.array_equal(dg["target_logit"][valid_d], zt[valid_d].astype(np.float32))
    assert np.array_equal(dg["draft_logit"][valid_d], zd[valid_d].astype(np.float32))
    draws = (dg["terminal_kind"] == ref["terminal_kind"]) & np.isin(ref["terminal_kind"], [1, 2, 3])
    assert draws.sum() > 0.9 * b.B
    S_gpu, S_ref = dg["terminal_mass"][draws], ref["resid_mass"][draws]
    assert np.all(np.abs(S_gpu - S_ref) <= 1e-5 * S_ref + 1e-7), np.max(np.abs(S_gpu - S_ref) / S_ref)
    bonus = draws & (ref["terminal_kind"] == 1)
    assert np.all(np.abs(dg["terminal_mass"][bonus] - 1.0) < 1e-5)


def test_diag_draft_logit_holds_q_with_probability_rows():
    rng = np.random.default_rng(5)
    b = W.with_qrows(W.make_random("qrows_diag", rng.integers(1, 7, size=24), 32000, "bf16", 1.0, 3.0, 1.0, 15, 25))
    acc, out, dg = run_gpu(b, diag=("draft_logit", "terminal_mass", "terminal_kind"))
    ref = run_oracle(b)
    assert compare_verdicts(acc, out, ref, b.cu, b.temperature)["n_hard"] == 0
    q_at = b.qrows[np.arange(b.n_draft_rows), b.tokens]
    assert np.array_equal(dg["draft_logit"], q_at)
    draws = (dg["terminal_kind"] == ref["terminal_kind"]) & np.isin(ref["terminal_kind"], [1, 2])
    assert np.all(np.abs(dg["terminal_mass"][draws] - ref["resid_mass"][draws]) <= 1e-5 * ref["resid_mass"][draws] + 1e-7)


def test_philox_uniforms_match_oracle_grid():
    import lossless_draft_verification_online_amd as sdv
    for seed, B, P in ((0, 3, 5), (0xFEEDFACECAFEBEEF, 257, 65), (2**64 - 1, 1, 1)):
        got = sdv.philox_uniforms(seed, B, P, device=DEV).cpu().numpy().view(np.uint32)
        assert np.array_equal(got, oracle.philox_grid(seed, B, P).reshape(B, P, 4)), (seed, B, P)


# ----------------------------------------------------------------------------- unstaged records
# The verdict kernel stages a request's chunk records in 48 KiB of shared memory when (rows x chunks)
# fits beside the residual masses; deeper requests on wide rows fold straight from the workspace.

@pytest.mark.parametrize("dtype,V,T,depths", [
    ("bf16", 600000, 1.0, [48, 3, 56, 0, 64]),     # 74 chunks: (2K + 1) 74 > 6070 staged records from K = 41
    ("bf16", 770000, 0.0, [64, 2, 60]),            # 94 chunks: (K + 1) 94 > 6050 at K = 64
    ("fp32", 200003, 1.0, [64, 1, 62]),            # 49 chunks, rows not of 16-byte length
])
def test_deep_requests_fold_from_the_workspace(dtype, V, T, depths):
    b = W.make_random(f"deep_{dtype}_{V}_T{T}", depths, V, dtype, T, 3.0, 0.15, data_seed=V + 31, verify_seed=V + 41)
    C = -(-V // (8192 if dtype == "bf16" else 4096))
    room = (48 * 1024 - C * 8) // 8
    rows = [(k + 1 if T == 0 else 2 * k + 1) * C for k in depths]
    assert max(rows) > room and min(rows) <= room  # both paths in one call
    _, _, ref, cmp, _ = check_parity(b)
    log(f"    excused {cmp['n_excused']}, accepted {ref['accepted_len'].tolist()}")
    if T == 0:
        assert cmp["n_excused"] == 0
