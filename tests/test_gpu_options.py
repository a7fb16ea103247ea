"""GPU parity of sdv_verify_opts: stop tokens and output budgets (SDCP "Verification and Commit",
step 7; M7.8 section 0x09), the caller's uniforms (SDCP Rule 2's HMAC-SHA-256 values from
sdv_sdcp_uniforms, strict test r < p/q), alone and combined with per-request profiles.

Verdicts, emitted counts and emitted tokens must match the fp64 oracle given the same options, up
to counted near-ties; requests whose emission ends inside the accepted drafts draw nothing.
"""
import json
import os

import numpy as np
import pytest
import torch

import lossless_draft_verification_online_amd as sdv
import workloads as W
from gpu_helpers import DEV, log, profile_args, to_device
from oracle import oracle
from oracle.compare import compare_verdicts

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _options(b, rng, stops=True, budget=True, sdcp=False):
    opts = {}
    if stops:
        lists = [list(rng.choice(b.V, size=rng.integers(0, 4), replace=False)) for _ in range(b.B)]
        # make stops likely: a quarter of the requests stop at one of their own draft tokens
        for i in range(b.B):
            K = b.cu[i + 1] - b.cu[i]
            if K and rng.random() < 0.25:
                lists[i].append(int(b.tokens[b.cu[i] + rng.integers(0, K)]))
        opts["stop_lists"] = oracle.stop_csr(lists)
    if budget:
        opts["budget"] = rng.integers(-1, 10, size=b.B).astype(np.int32)
    if sdcp:
        seeds = rng.integers(0, 2**63, size=b.B, dtype=np.int64).astype(np.uint64)
        sessions = rng.integers(0, 256, size=(b.B, 16), dtype=np.uint8)
        rounds = rng.integers(0, 1000, size=b.B).astype(np.uint32)
        opts["accept_uniform"], opts["draw_uniform"] = sdv.sdcp_uniforms(b.cu, seeds, sessions, rounds)
    return opts


def _run_both(b, opts, diag=("terminal_kind",)):
    ins = (to_device(b.target, b.dtype), to_device(b.draft, b.dtype), torch.from_numpy(b.tokens).to(DEV),
           torch.from_numpy(b.cu).to(DEV))
    temperature, seed = profile_args(b)
    kw = {}
    if "stop_lists" in opts:
        offs, toks = opts["stop_lists"]
        kw["stop_offsets"] = torch.from_numpy(offs).to(DEV)
        kw["stop_tokens"] = torch.from_numpy(toks).to(DEV)
    if "budget" in opts:
        kw["budget"] = torch.from_numpy(opts["budget"]).to(DEV)
    if "accept_uniform" in opts:
        kw["accept_uniform"] = torch.from_numpy(opts["accept_uniform"]).to(DEV)
        kw["draw_uniform"] = torch.from_numpy(opts["draw_uniform"]).to(DEV)
    acc, out, extra = sdv.verify_ex(*ins, temperature, seed, diag=diag, **kw)
    torch.cuda.synchronize()
    t_or = b.temp_each.astype(np.float64) if b.temp_each is not None else b.temperature
    s_or = b.seed_each if b.seed_each is not None else b.seed
    ref = oracle.verify(b.target, b.draft, b.tokens, b.cu, t_or, s_or, diag=True, **opts)
    got = {k: v.cpu().numpy() for k, v in extra.items()}
    return acc.cpu().numpy(), out.cpu().numpy(), got, ref, t_or


def _check(b, opts):
    acc, out, got, ref, t_or = _run_both(b, opts)
    cmp = compare_verdicts(acc, out, ref, b.cu, t_or)
    assert cmp["n_hard"] == 0, cmp["hard"][:5]
    ok = np.ones(b.B, dtype=bool)
    for i, _ in cmp["excused"]:
        ok[i] = False
    if "stop_lists" in opts or "budget" in opts:
        assert np.array_equal(got["emitted_len"][ok], ref["emitted_len"][ok])
    assert np.array_equal(got["terminal_kind"][ok], ref["terminal_kind"][ok])
    log(f"  {b.name}: {cmp['n_excused']} near-tie excuses, "
        f"{int((ref['terminal_kind'] == oracle.TERM_NONE).sum())} requests stopped inside their drafts")
    return acc, out, got, ref


@pytest.mark.parametrize("T", [0.0, 0.9])
def test_stops_and_budgets_match_oracle(T):
    rng = np.random.default_rng(int(T * 10) + 1)
    b = W.make_random(f"stops_T{T}", rng.integers(0, 9, size=64), 20011, "bf16", T, 3.0, 1.0, data_seed=11,
                      verify_seed=12, keep_draft=True)
    _, _, _, ref = _check(b, _options(b, rng))
    assert (ref["terminal_kind"] == oracle.TERM_NONE).any()


def test_sdcp_uniforms_match_oracle():
    rng = np.random.default_rng(5)
    b = W.make_random("sdcp_uniforms", rng.integers(0, 9, size=64), 32000, "bf16", 1.0, 3.0, 1.5, data_seed=13,
                      verify_seed=0)
    _check(b, _options(b, rng, stops=False, budget=False, sdcp=True))


def test_everything_together_with_profiles():
    rng = np.random.default_rng(6)
    base = W.make_random("all_options", rng.integers(0, 9, size=96), 4099, "fp32", 1.0, 2.0, 1.0, data_seed=14,
                         verify_seed=0, keep_draft=True)
    t, s = W.mixed_profiles(base.B, rng)
    b = W.with_profiles(base, t, s, token_seed=15)
    _check(b, _options(b, rng, stops=True, budget=True, sdcp=True))


def test_full_size_b256_with_stops_budgets_and_sdcp_uniforms():
    rng = np.random.default_rng(7)
    b = W.ragged_b256()
    _check(b, _options(b, rng, stops=True, budget=True, sdcp=True))


def test_m78_stopping_example_on_the_gpu():
    g = json.load(open(os.path.join(GOLDEN, "m78_stopping.json")))
    P, K = g["P"], g["K"]
    drafts, bonus = [3, 8, 1, 12], 6
    rng = np.random.default_rng(0)
    rows = rng.standard_normal((K + 1, 16)).astype(np.float32)
    for r, x in enumerate(drafts + [bonus]):
        rows[r, x] = rows[r].max() + 1.0
    b = W.Batch(name="m78", V=16, dtype="fp32", temperature=0.0, seed=0, target=rows, draft=None,
                tokens=np.array(drafts, dtype=np.int32), cu=W.offsets_from_depths([K]))
    for case in g["cases"]:
        opts = {"stop_lists": oracle.stop_csr([[bonus]] if case["stop_at_bonus"] else [[]])}
        if case["budget"] is not None:
            opts["budget"] = np.array([case["budget"]], dtype=np.int32)
        acc, out, got, ref = _check(b, opts)
        n = int(got["emitted_len"][0])
        E, F = min(n, K), int(n == K + 1)
        assert [P + E + F, P + E, P + min(E, K - 1)] == case["expect"], case["what"]


def test_malformed_stop_list_rejects_only_its_request():
    b = W.make_random("bad_stops", [2, 3, 1, 4], 64, "fp32", 1.0, 2.0, 1.0, data_seed=16, verify_seed=17)
    offs = np.array([0, 1, 0, 2, 2], dtype=np.int32)  # request 1's list runs backwards
    toks = np.array([5, 6], dtype=np.int32)
    acc, out, got, ref = _check(b, {"stop_lists": (offs, toks)})
    assert acc[1] == -1 and got["emitted_len"][1] == 0
    assert (out[b.cu[1] + 1: b.cu[2] + 2] == -1).all()
