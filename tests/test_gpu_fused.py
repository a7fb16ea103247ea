"""The fused path (one kernel: stream, verdicts and draws, with corrections shared among waves)
against the two-kernel path and the oracle.

Both paths take the same decisions from the same records in the same arithmetic, so their outputs
must agree bit for bit, diagnostics included.  The one exception: at rows of one chunk the
two-kernel path totals a correction's weights inside its in-chunk search, so its tokens may differ
where u * S falls within rounding of a CDF step; there both are compared with the oracle instead.
"""
import numpy as np
import pytest
import torch

import lossless_draft_verification_online_amd as sdv
import workloads as W
from gpu_helpers import DEV, log, profile_args, run_oracle, upload
from oracle.compare import compare_verdicts

pytestmark = pytest.mark.gpu

DIAG_SAMPLING = ("target_lse", "draft_lse", "ratio", "accept_uniform", "draw_uniform", "terminal_kind",
                 "target_logit", "draft_logit", "terminal_mass")
DIAG_GREEDY = ("target_argmax", "terminal_kind")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(b, path, ins=None, **kw):
    t, d, x, cu = upload(b) if ins is None else ins
    temperature, seed = profile_args(b)
    diag = DIAG_GREEDY if b.temperature == 0 else DIAG_SAMPLING
    acc, out, dg = sdv.verify_ex(t, d, x, cu, temperature, seed, diag=diag, verdict_path=path, **kw)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy(), {k: v.cpu().numpy() for k, v in dg.items()}


def _same(a, b, name):
    assert np.array_equal(a[0], b[0]), f"{name}: accepted lengths differ"
    assert np.array_equal(a[1], b[1]), f"{name}: tokens differ at {np.nonzero(a[1] != b[1])[0][:10]}"
    for k in a[2]:
        x, y = a[2][k], b[2][k]
        same = (x == y) | (np.isnan(x) & np.isnan(y)) if x.dtype.kind == "f" else (x == y)
        assert same.all(), f"{name}: diag {k} differs at {np.nonzero(~same)[0][:10]}"


CASES = [
    ("ragged_bf16_32000", lambda rng: W.make_random("ragged_bf16_32000", rng.integers(0, 9, 64), 32000, "bf16", 1.0,
                                                    3.0, rng.uniform(0.5, 3.0, 64), 101, 201)),
    ("ragged_bf16_151936_T07", lambda rng: W.make_random("ragged_bf16_151936_T07", rng.integers(0, 9, 48), 151936,
                                                         "bf16", 0.7, 3.0, rng.uniform(0.5, 3.0, 48), 102, 202)),
    ("ragged_fp32_20000", lambda rng: W.make_random("ragged_fp32_20000", rng.integers(0, 12, 40), 20000, "fp32", 1.2,
                                                    2.0, 1.0, 103, 203)),
    ("partial_last_chunk_bf16", lambda rng: W.make_random("partial_last_chunk_bf16", rng.integers(0, 6, 30), 20008,
                                                          "bf16", 1.0, 3.0, 1.5, 104, 204)),
    ("greedy_bf16_151936", lambda rng: W.make_random("greedy_bf16_151936", rng.integers(0, 9, 80), 151936, "bf16", 0.0,
                                                     4.0, 1.0, 105, 205)),
    ("greedy_fp32_5000", lambda rng: W.make_random("greedy_fp32_5000", rng.integers(0, 9, 33), 5000, "fp32", 0.0, 4.0,
                                                   0.5, 106, 206)),
    ("deep_bf16_40000", lambda rng: W.make_random("deep_bf16_40000", rng.integers(30, 65, 6), 40000, "bf16", 1.0, 3.0,
                                                  0.1, 107, 207)),
    ("wide_fp32_300000", lambda rng: W.make_random("wide_fp32_300000", rng.integers(0, 5, 6), 300000, "fp32", 1.0, 3.0,
                                                   2.0, 108, 208)),
]


@pytest.mark.parametrize("name", [c[0] for c in CASES])
def test_fused_equals_two_kernel_path(name):
    b = dict(CASES)[name](np.random.default_rng(len(name)))
    log(f"  fused vs two-kernel {b.name}: B={b.B} n_d={b.n_draft_rows} V={b.V} {b.dtype} T={b.temperature}")
    ins = upload(b)
    fused = _run(b, 0, ins)
    two = _run(b, 1, ins)
    _same(fused, two, b.name)
    ref = run_oracle(b)
    cmp = compare_verdicts(fused[0], fused[1], ref, b.cu, b.temperature)
    assert cmp["n_hard"] == 0, cmp["hard"][:10]


def test_fused_one_chunk_rows_against_oracle():
    """Rows of one chunk (V = 1000, binary32): tokens against the oracle."""
    rng = np.random.default_rng(9)
    for rnd in range(4):
        b = W.make_random(f"one_chunk_{rnd}", rng.integers(0, 8, 128), 1000, "fp32", 1.0, 2.0, 1.0, 300 + rnd, 400 + rnd)
        acc, out, dg = _run(b, 0)
        ref = run_oracle(b)
        cmp = compare_verdicts(acc, out, ref, b.cu, b.temperature)
        assert cmp["n_hard"] == 0, cmp["hard"][:10]


def test_fused_options_and_bad_requests():
    """Stop lists, budgets, caller uniforms and rejected requests, fused against two-kernel."""
    rng = np.random.default_rng(17)
    depths = rng.integers(0, 9, 40)
    depths[1], depths[2], depths[5] = 3, 3, 0
    b = W.make_random("fused_options", depths, 24000, "bf16", 1.0, 3.0, rng.uniform(0.3, 2.0, 40), 111, 211)
    b.tokens = b.tokens.copy()
    b.tokens[b.cu[1] + 1] = 24000  # request 1: a token out of range
    d = W.bf16_to_f32(b.draft).copy()
    d[b.cu[2], b.tokens[b.cu[2]]] = -np.inf  # request 2: q(x) = 0
    b.draft = W.bf16_bits(d)
    ins = upload(b)
    B, n_d = b.B, b.n_draft_rows
    stop_off = np.zeros(B + 1, np.int32)
    stops = []
    for i in range(B):
        lst = [int(b.tokens[b.cu[i] + 1])] if (i % 3 == 0 and depths[i] > 1) else []
        stops += lst
        stop_off[i + 1] = len(stops)
    kw = dict(stop_offsets=torch.from_numpy(stop_off).to(DEV),
              stop_tokens=torch.tensor(stops, dtype=torch.int32, device=DEV),
              budget=torch.from_numpy(rng.integers(-1, 10, B).astype(np.int32)).to(DEV))
    _same(_run(b, 0, ins, **kw), _run(b, 1, ins, **kw), "stops_and_budget")
    r = torch.from_numpy(rng.random(n_d)).to(DEV)
    u = torch.from_numpy(rng.random(n_d + B)).to(DEV)
    fused = _run(b, 0, ins, accept_uniform=r, draw_uniform=u)
    _same(fused, _run(b, 1, ins, accept_uniform=r, draw_uniform=u), "caller_uniforms")
    assert fused[0][1] == -1 and fused[0][2] == -1 and fused[0][5] >= 0


def test_fused_depth_limit_and_malformed_offsets():
    b = W.make_random("fused_limit", [65, 2, 0, 3], 4096, "fp32", 1.0, 1.0, 1.0, 5, 6)
    t, d, x, cu = upload(b)
    for path in (0, 1):
        out = torch.full((b.n_draft_rows + b.B,), -7, dtype=torch.int32, device=DEV)
        acc = torch.full((b.B,), -9, dtype=torch.int32, device=DEV)
        sdv.verify_ex(t, d, x, cu, 1.0, 6, out=(acc, out), verdict_path=path)
        torch.cuda.synchronize()
        a = acc.cpu().numpy()
        assert a[0] == -1 and (a[1:] >= 0).all(), (path, a)
        assert (out[:66].cpu().numpy() == -7).all()
    bad_cu = cu.clone()
    bad_cu[2] = bad_cu[1] - 1  # decreasing offsets: every request rejected, no slot written
    for path in (0, 1):
        out = torch.full((b.n_draft_rows + b.B,), -7, dtype=torch.int32, device=DEV)
        acc = torch.full((b.B,), -9, dtype=torch.int32, device=DEV)
        sdv.verify_ex(t, d, x, bad_cu, 1.0, 6, out=(acc, out), verdict_path=path)
        torch.cuda.synchronize()
        assert (acc.cpu().numpy() == -1).all() and (out.cpu().numpy() == -7).all(), path


def test_fused_headline_batch_repeated():
    """The 256 x 128256 bf16 ragged batch, 24 calls on one workspace with fresh seeds: every call
    equal to the two-kernel path (8 of them also checked against the oracle)."""
    b = W.ragged_b256()
    ins = upload(b)
    for rnd in range(24):
        b.seed = 4000 + rnd
        fused = _run(b, 0, ins)
        if rnd % 3 == 0:
            _same(fused, _run(b, 1, ins), f"ragged_b256 seed {b.seed}")
            ref = run_oracle(b)
            cmp = compare_verdicts(fused[0], fused[1], ref, b.cu, b.temperature)
            assert cmp["n_hard"] == 0, cmp["hard"][:10]
        log(f"    seed {b.seed}: accepted {int(fused[0].sum())}")


def test_fused_greedy_headline_batch():
    b = W.greedy_b512()
    ins = upload(b)
    fused = _run(b, 0, ins)
    _same(fused, _run(b, 1, ins), "greedy_b512")
    ref = run_oracle(b)
    cmp = compare_verdicts(fused[0], fused[1], ref, b.cu, b.temperature)
    assert cmp["n_hard"] == 0 and cmp["n_excused"] == 0
