"""The verdict pass with several workgroups per request (sdv_options.verdict_split): the workgroups
of a request share a correction's residual pass, each taking a range of chunks, and the last to
finish draws.  A chunk's mass is computed the same way whichever workgroup computes it, so every
output is bit-identical whatever the split: checked against one workgroup per request across the
rules and inputs the verdict kernel takes (aligned and unaligned rows, bf16 and fp32, a partial
last chunk, depth 0, q rows, top-k / top-p, per-request profiles, bad proposals), and the automatic
split of a small batch of wide rows against the oracle."""
import numpy as np
import pytest
import torch

import lossless_draft_verification_online_amd as sdv
import workloads as W
from gpu_helpers import DEV, check_parity, log, profile_args, upload

pytestmark = pytest.mark.gpu

DIAG = ("terminal_kind", "draw_uniform", "target_lse", "ratio")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(b, split, dev_inputs):
    t, d, x, cu = dev_inputs
    temperature, seed = profile_args(b)
    kw = {}
    if b.qrows is not None:
        kw["draft_probs"] = torch.from_numpy(b.qrows).to(DEV)
    if b.top_k is not None:
        kw["top_k"] = torch.from_numpy(b.top_k).to(DEV)
        kw["top_p_milli"] = torch.from_numpy(b.top_p_milli).to(DEV)
    acc, out, dg = sdv.verify_ex(t, d, x, cu, temperature, seed, diag=DIAG, verdict_split=split, **kw)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy(), {k: v.cpu().numpy() for k, v in dg.items()}


def _same_for_every_split(b, splits):
    dev_inputs = upload(b)
    C = -(-b.V // (8192 if b.dtype == "bf16" else 4096))
    ref = _run(b, 1, dev_inputs)
    corrections = int((ref[2]["terminal_kind"] == 2).sum())
    log(f"  {b.name}: B={b.B} V={b.V} {b.dtype} C={C}, {corrections} corrections, splits {splits}")
    assert corrections > 0
    for s in splits:
        got = _run(b, s, dev_inputs)
        np.testing.assert_array_equal(got[0], ref[0], err_msg=f"accepted_len, split {s}")
        np.testing.assert_array_equal(got[1], ref[1], err_msg=f"out_tokens, split {s}")
        for k in DIAG:
            np.testing.assert_array_equal(got[2][k], ref[2][k], err_msg=f"{k}, split {s}")


@pytest.mark.parametrize("V,dtype", [(65536, "bf16"), (65537, "bf16"), (40000, "fp32"), (20011, "fp32")])
def test_split_outputs_are_bit_identical(V, dtype):
    rng = np.random.default_rng(V)
    depths = rng.integers(0, 9, size=48)
    depths[:3] = 0
    b = W.make_random(f"split_{dtype}_{V}", depths, V, dtype, 1.0, 3.0, rng.uniform(0.5, 3.0, size=48),
                      data_seed=V + 3, verify_seed=V)
    bad = int(np.nonzero(b.depths >= 2)[0][0])
    b.tokens[b.cu[bad] + 1] = -3  # a bad proposal: that request alone is rejected
    C = -(-V // (8192 if dtype == "bf16" else 4096))
    _same_for_every_split(b, sorted({2, 3, C - 1, C, C + 5}))


@pytest.mark.parametrize("V,dtype", [(65536, "bf16"), (65537, "bf16"), (40000, "fp32")])
def test_split_with_q_rows(V, dtype):
    rng = np.random.default_rng(5)
    b = W.with_qrows(W.make_random(f"split_q_{dtype}_{V}", rng.integers(0, 9, size=40), V, dtype, 0.9, 3.0, 1.5,
                                   data_seed=51, verify_seed=52))
    C = -(-V // (8192 if dtype == "bf16" else 4096))
    _same_for_every_split(b, sorted({2, 3, C}))


def test_split_with_top_k_top_p():
    rng = np.random.default_rng(6)
    b = W.make_random("split_trunc", rng.integers(0, 9, size=40), 65536, "bf16", 1.0, 3.0,
                      rng.uniform(0.5, 2.0, size=40), data_seed=61, verify_seed=62, keep_draft=True)
    _same_for_every_split(W.with_truncation(b, 200, 950), [2, 5, 8])


def test_split_with_profiles():
    rng = np.random.default_rng(7)
    base = W.make_random("split_prof", rng.integers(0, 9, size=64), 40000, "fp32", 1.0, 3.0, 1.5, data_seed=71,
                         verify_seed=0, keep_draft=True)
    t, s = W.mixed_profiles(base.B, rng, temps=(0.0, 0.8, 1.2))
    _same_for_every_split(W.with_profiles(base, t, s, token_seed=72), [2, 4, 10])


def test_automatic_split_of_a_small_batch_matches_oracle():
    # B = 3 requests of 128256-token rows: 16 chunks per row, four workgroups per request
    rng = np.random.default_rng(8)
    b = W.make_random("split_auto_b3", [4, 0, 7], 128256, "bf16", 1.0, 3.0, 1.5, data_seed=81, verify_seed=82)
    for seed in range(4):
        check_parity(b, seed=int(rng.integers(0, 2**62)))


def test_split_counters_restart_every_call():
    # one workspace, filled with 0xff bytes first, for calls of two shapes: the row pass of every
    # call zeroes the counters, so stale or garbage counts never decide which workgroup draws
    rng = np.random.default_rng(9)
    b1 = W.make_random("split_ws_a", [4, 7, 2], 65536, "bf16", 1.0, 3.0, 1.5, data_seed=91, verify_seed=92)
    b2 = W.make_random("split_ws_b", rng.integers(1, 9, size=5), 98304, "bf16", 1.0, 3.0, 1.5, data_seed=93,
                       verify_seed=94)
    need = max(int(sdv._native.lib().sdv_workspace_bytes(b.B, b.n_draft_rows, b.V, 0)) for b in (b1, b2))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    inputs = {b.name: upload(b) for b in (b1, b2)}
    fresh = {b.name: _run(b, 1, inputs[b.name]) for b in (b1, b2)}

    def shared(b, split):
        t, d, x, cu = inputs[b.name]
        acc, out, dg = sdv.verify_ex(t, d, x, cu, b.temperature, b.seed, diag=DIAG, verdict_split=split, workspace=ws)
        torch.cuda.synchronize()
        return acc.cpu().numpy(), out.cpu().numpy(), {k: v.cpu().numpy() for k, v in dg.items()}
    for b, split in [(b1, 8), (b2, 3), (b1, 2), (b2, 12), (b1, 8)]:
        got, ref = shared(b, split), fresh[b.name]
        np.testing.assert_array_equal(got[0], ref[0])
        np.testing.assert_array_equal(got[1], ref[1])
        for k in DIAG:
            np.testing.assert_array_equal(got[2][k], ref[2][k])
    log(f"  shared workspace: {need} bytes, {int((fresh[b1.name][2]['terminal_kind'] == 2).sum())} + "
        f"{int((fresh[b2.name][2]['terminal_kind'] == 2).sum())} corrections")
