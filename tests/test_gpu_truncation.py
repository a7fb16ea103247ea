"""GPU parity of top-k / top-p sampling profiles (SDCP, section "Session Contract": temperature, then
top-k, then top-p) through sdv_verify_opts.

Per row, the number of kept tokens must equal the oracle's exactly; verdicts must equal the
oracle's up to counted near-ties.  Top-p cuts within 1e-6 of their threshold (relative to the
top-k mass) are excused, as every other floating-point decision is.  Draft tokens are drawn from
the drafter's truncated distribution, so that proposals are valid: the test redraws each
position's token over the kept set the oracle computes (tests may call the oracle; the input
generator stays free of the method's arithmetic).  A few positions then get a token outside the
kept set on purpose: the oracle and the kernel must both reject that request.
"""
import numpy as np
import pytest
import torch

import lossless_draft_verification_online_amd as sdv
import workloads as W
from gpu_helpers import DEV, log, to_device
from oracle import oracle
from oracle.compare import compare_verdicts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _temps(b):
    return b.temp_each.astype(np.float64) if b.temp_each is not None else np.full(b.B, b.temperature)


def drafter_tokens(b, top_k, milli, rng, n_bad=0):
    """Tokens drawn by the drafter from its truncated rows (Gumbel-max over the kept set); the first
    n_bad sampled requests get one token outside the kept set instead."""
    T = _temps(b)
    tokens = b.tokens.copy()
    bad_left = n_bad
    for i in range(b.B):
        if not T[i] > 0 or top_k[i] < 0 or not 0 <= milli[i] <= 1000:
            continue
        for j in range(int(b.depths[i])):
            d = int(b.cu[i]) + j
            row = b.draft[d]
            keep = oracle.truncate_row(row, T[i], int(top_k[i]), int(milli[i]))["keep"]
            z = (W.bf16_to_f32(row) if b.dtype == "bf16" else row).astype(np.float64)
            g = -np.log(-np.log(rng.random(z.shape)))
            tokens[d] = int(np.argmax(np.where(keep, z / T[i] + g, -np.inf)))
            if bad_left > 0 and j == 0 and not keep.all():
                tokens[d] = int(np.nonzero(~keep)[0][0])
                bad_left -= 1
    return tokens.astype(np.int32)


def run_both(b, top_k, milli, diag=("terminal_kind", "target_lse", "kept_tokens")):
    t, d = to_device(b.target, b.dtype), to_device(b.draft, b.dtype)
    x, cu = torch.from_numpy(b.tokens).to(DEV), torch.from_numpy(b.cu).to(DEV)
    kw = {"top_k": torch.from_numpy(np.asarray(top_k, dtype=np.int32)).to(DEV),
          "top_p_milli": torch.from_numpy(np.asarray(milli, dtype=np.int32)).to(DEV)}
    if b.qrows is not None:
        kw["draft_probs"] = torch.from_numpy(b.qrows).to(DEV)
        d = None
    if b.temp_each is not None:
        temperature = torch.from_numpy(b.temp_each.astype(np.float32)).to(DEV)
        seed = torch.from_numpy(b.seed_each.astype(np.uint64).view(np.int64)).to(DEV)
    else:
        temperature, seed = b.temperature, b.seed
    acc, out, extra = sdv.verify_ex(t, d, x, cu, temperature, seed, diag=diag, **kw)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in extra.items()}
    t_or = b.temp_each.astype(np.float64) if b.temp_each is not None else b.temperature
    s_or = b.seed_each if b.seed_each is not None else b.seed
    okw = {} if b.qrows is None else {"draft_probs": b.qrows}
    ref = oracle.verify(b.target, b.draft if b.qrows is None else None, b.tokens, b.cu, t_or, s_or, diag=True,
                        top_k=top_k, top_p_milli=milli, **okw)
    return acc.cpu().numpy(), out.cpu().numpy(), got, ref


def check(b, top_k, milli, expect_bad=None):
    log(f"  truncation {b.name}: B={b.B} n_draft_rows={b.n_draft_rows} V={b.V} {b.dtype}")
    acc, out, got, ref = run_both(b, top_k, milli)
    T = _temps(b)
    cmp = compare_verdicts(acc, out, ref, b.cu, T)
    assert cmp["n_hard"] == 0, cmp["hard"][:5]
    # kept counts: every row of a request the oracle truncated (T > 0, valid profile, tokens in range)
    n_t = b.n_draft_rows + b.B
    rows = []
    for i in range(b.B):
        if not T[i] > 0 or top_k[i] < 0 or not 0 <= milli[i] <= 1000:
            continue
        lo, hi = int(b.cu[i]), int(b.cu[i + 1])
        if ((b.tokens[lo:hi] < 0) | (b.tokens[lo:hi] >= b.V)).any():
            continue
        rows += list(range(lo + i, hi + i + 1))
        if b.qrows is None:
            rows += [n_t + d for d in range(lo, hi)]
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size:
        sure = ref["filter_margin"][rows] >= 1e-6
        assert np.array_equal(got["kept_tokens"][rows][sure], ref["kept_tokens"][rows][sure]), \
            np.nonzero(got["kept_tokens"][rows] != ref["kept_tokens"][rows])[0][:10]
    ok = np.ones(b.B, dtype=bool)
    for i, _ in cmp["excused"]:
        ok[i] = False
    assert np.array_equal(got["terminal_kind"][ok], ref["terminal_kind"][ok])
    # the kept-mass LSE of every target row of a valid sampling request, within 1e-5 relative
    tr = [r for i in range(b.B) if T[i] > 0 and acc[i] >= 0 and ok[i]
          for r in range(int(b.cu[i]) + i, int(b.cu[i + 1]) + i + 1)]
    if tr:
        np.testing.assert_allclose(got["target_lse"][tr], ref["target_lse"][tr], rtol=1e-5, atol=1e-5)
    if expect_bad is not None:
        assert (ref["accepted_len"][expect_bad] == -1).all()
    log(f"    {cmp['n_excused']} excused, {int((acc == -1).sum())} rejected, "
        f"mean kept {float(np.mean(ref['kept_tokens'][rows])) if rows.size else float('nan'):.1f}")
    return acc, out, got, ref


def _profiles(B, V, rng):
    top_k = rng.choice([0, 1, 2, 5, 50, 1000, V, V + 7], size=B).astype(np.int32)
    milli = rng.choice([1000, 1000, 950, 900, 500, 100, 0], size=B).astype(np.int32)
    return top_k, milli


@pytest.mark.parametrize("dtype,V", [("bf16", 32000), ("fp32", 4099), ("bf16", 1000), ("bf16", 1001),
                                     ("bf16", 20011)])
def test_mixed_profiles_match_oracle(dtype, V):
    rng = np.random.default_rng(V)
    base = W.make_random(f"trunc_{dtype}_{V}", rng.integers(0, 9, size=64), V, dtype, 1.0, 3.0,
                         rng.uniform(0.5, 3.0, size=64), data_seed=V + 1, verify_seed=V + 2, keep_draft=True)
    t, s = W.mixed_profiles(base.B, rng)
    b = W.with_profiles(base, t, s, token_seed=V + 3)
    top_k, milli = _profiles(b.B, V, rng)
    b.tokens = drafter_tokens(b, top_k, milli, rng, n_bad=3)
    check(b, top_k, milli)


@pytest.mark.parametrize("V", [20000, 20001])
def test_ties_everywhere(V):
    """Logits rounded to a few values: every cut lands inside a group of equal logits, so the kept
    copies are decided by token id (and the kernel's search for the last kept id is exercised), on
    16-byte rows and on rows split at 16-byte boundaries."""
    rng = np.random.default_rng(41)
    B = 48
    depths = rng.integers(0, 6, size=B)
    cu = W.offsets_from_depths(depths)
    n_d = int(cu[-1])
    tgt = np.round(rng.standard_normal((n_d + B, V)) * 1.5).astype(np.float32)
    drf = np.round(rng.standard_normal((n_d, V)) * 1.5).astype(np.float32)
    b = W.Batch(name="ties", V=V, dtype="bf16", temperature=0.9, seed=5, target=W.bf16_bits(tgt),
                draft=W.bf16_bits(drf), tokens=np.zeros(n_d, dtype=np.int32), cu=cu)
    top_k = rng.choice([1, 3, 100, 2500, 7001], size=B).astype(np.int32)
    milli = rng.choice([1000, 800, 300, 0], size=B).astype(np.int32)
    b.tokens = drafter_tokens(b, top_k, milli, rng)
    check(b, top_k, milli)


def test_constant_rows_full_width():
    """Every logit equal (V = 128256): top-k keeps the smallest ids, and top-p over equal masses is
    exact (the nucleus of mass m/1000 holds ceil(m/1000 * kept) tokens)."""
    B, V, K = 6, 128256, 2
    cu = W.offsets_from_depths(np.full(B, K))
    n_d = B * K
    target = np.full((n_d + B, V), W.bf16_bits(np.float32(0.5)), dtype=np.uint16)
    draft = np.full((n_d, V), W.bf16_bits(np.float32(-1.25)), dtype=np.uint16)
    top_k = np.array([5000, 0, 70000, 1, 128255, 3], dtype=np.int32)
    milli = np.array([1000, 500, 250, 1000, 999, 0], dtype=np.int32)
    tokens = np.array([3, 4000, 1, 60000, 20000, 64000, 0, 0, 100, 128254, 0, 1], dtype=np.int32)
    b = W.Batch(name="constant", V=V, dtype="bf16", temperature=1.0, seed=9, target=target, draft=draft,
                tokens=tokens, cu=cu)
    acc, out, got, ref = check(b, top_k, milli)
    # kept: top-5000; half of 128256; a quarter of the top 70000; top-1; ceil(0.999 * 128255); the
    # first of the top 3
    want = [5000, 64128, 17500, 1, 128127, 1]
    for i in range(B):
        assert got["kept_tokens"][int(cu[i]) + i] == want[i]
        assert got["kept_tokens"][n_d + B + int(cu[i])] == want[i]
    # equal kept probabilities give ratio 1 (both drafts accepted); requests 2, 4 and 5 propose a
    # token their draft rows do not keep
    assert acc.tolist() == [2, 2, -1, 2, -1, -1]


def test_rows_with_minus_infinity():
    """Masked vocabularies: -inf logits rank last; top-k larger than the finite count keeps some of
    them at zero probability."""
    rng = np.random.default_rng(43)
    B, V = 16, 3000
    depths = rng.integers(1, 5, size=B)
    cu = W.offsets_from_depths(depths)
    n_d = int(cu[-1])
    tgt = (rng.standard_normal((n_d + B, V)) * 2).astype(np.float32)
    drf = (rng.standard_normal((n_d, V)) * 2).astype(np.float32)
    tgt[:, 2000:] = -np.inf
    drf[:, 2500:] = -np.inf
    b = W.Batch(name="masked", V=V, dtype="fp32", temperature=1.2, seed=3, target=tgt, draft=drf,
                tokens=np.zeros(n_d, dtype=np.int32), cu=cu)
    top_k = rng.choice([10, 1999, 2200, 2999], size=B).astype(np.int32)
    milli = rng.choice([1000, 990], size=B).astype(np.int32)
    b.tokens = drafter_tokens(b, top_k, milli, rng)
    check(b, top_k, milli)


def test_top_k_one_equals_the_greedy_rule_on_the_gpu():
    rng = np.random.default_rng(47)
    b = W.make_random("topk1", rng.integers(0, 9, size=96), 32000, "bf16", 0.0, 3.0, 0.7, data_seed=48,
                      verify_seed=49, keep_draft=True)
    ins = (to_device(b.target, b.dtype), to_device(b.draft, b.dtype), torch.from_numpy(b.tokens).to(DEV),
           torch.from_numpy(b.cu).to(DEV))
    g_acc, g_out, _ = sdv.verify_ex(*ins, 0.0, 0)
    ones = torch.ones(b.B, dtype=torch.int32, device=DEV)
    for T in (0.5, 1.0, 2.0):
        acc, out, extra = sdv.verify_ex(*ins, T, 11, top_k=ones, diag=("kept_tokens",))
        torch.cuda.synchronize()
        assert torch.equal(acc, g_acc) and torch.equal(out, g_out)
        assert (extra["kept_tokens"] == 1).all()


def test_given_probability_rows_with_truncated_target():
    rng = np.random.default_rng(53)
    base = W.make_random("trunc_q", rng.integers(0, 7, size=48), 16000, "bf16", 1.0, 3.0, 1.0, data_seed=54,
                         verify_seed=55, keep_draft=True)
    b = W.with_qrows(base)
    top_k = rng.choice([0, 20, 400], size=b.B).astype(np.int32)
    milli = rng.choice([1000, 900], size=b.B).astype(np.int32)
    check(b, top_k, milli)


def test_invalid_profiles_reject_only_their_requests():
    rng = np.random.default_rng(59)
    base = W.make_random("bad_trunc", rng.integers(0, 5, size=32), 2048, "bf16", 1.0, 3.0, 1.0, data_seed=60,
                         verify_seed=61, keep_draft=True)
    t, s = W.mixed_profiles(base.B, rng, temps=(0.0, 1.0))
    b = W.with_profiles(base, t, s, token_seed=62)
    top_k = np.zeros(b.B, dtype=np.int32)
    milli = np.full(b.B, 1000, dtype=np.int32)
    top_k[[1, 2]] = -1
    milli[[5, 6]] = [1001, -3]
    acc, out, got, ref = check(b, top_k, milli, expect_bad=[1, 2, 5, 6])
    assert (acc[[1, 2, 5, 6]] == -1).all()


def test_full_size_b256_top_k_50_top_p_0_9():
    rng = np.random.default_rng(67)
    b = W.ragged_b256()
    top_k = np.full(b.B, 50, dtype=np.int32)
    milli = np.full(b.B, 900, dtype=np.int32)
    b.tokens = drafter_tokens(b, top_k, milli, rng)
    check(b, top_k, milli)


def test_cuts_below_the_window_take_the_radix_select():
    """bf16 rows whose cut lies below the 4096 keys under the maximum: a top-k larger than the
    window holds, and nuclei that reach deep into the tail at a high temperature.  These rows go
    through the exact radix select (16-byte rows, the vector path)."""
    rng = np.random.default_rng(71)
    B, V = 24, 32000
    depths = rng.integers(1, 5, size=B)
    cu = W.offsets_from_depths(depths)
    n_d = int(cu[-1])
    tgt = (rng.standard_normal((n_d + B, V)) * 4).astype(np.float32)
    drf = (tgt[np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(B)])]
           + rng.standard_normal((n_d, V))).astype(np.float32)
    b = W.Batch(name="below_window", V=V, dtype="bf16", temperature=6.0, seed=21, target=W.bf16_bits(tgt),
                draft=W.bf16_bits(drf), tokens=np.zeros(n_d, dtype=np.int32), cu=cu)
    top_k = rng.choice([20000, 31000, 0], size=B).astype(np.int32)
    milli = rng.choice([1000, 999, 995], size=B).astype(np.int32)
    milli[top_k == 0] = 999  # top-p alone, over a flat distribution
    b.tokens = drafter_tokens(b, top_k, milli, rng)
    acc, out, got, ref = check(b, top_k, milli)
    # the cut of every truncated row lies below the window: fewer than 4096 distinct keys cannot hold it
    assert (ref["kept_tokens"][: n_d + B] > 16000).all()


@pytest.mark.parametrize("V", [32000, 128256])
def test_binary32_rows_on_the_vector_path(V):
    """binary32 rows of 16-byte length: the radix select over three digit levels, vector loads."""
    rng = np.random.default_rng(V + 73)
    base = W.make_random(f"trunc_fp32_{V}", rng.integers(0, 7, size=32), V, "fp32", 1.0, 3.0,
                         rng.uniform(0.5, 3.0, size=32), data_seed=V + 74, verify_seed=V + 75, keep_draft=True)
    t, s = W.mixed_profiles(base.B, rng)
    b = W.with_profiles(base, t, s, token_seed=V + 76)
    top_k, milli = _profiles(b.B, V, rng)
    b.tokens = drafter_tokens(b, top_k, milli, rng, n_bad=2)
    check(b, top_k, milli)


def _counted_row(kind, V, rng):
    """Rows for the row pass's per-chunk key counts (bf16, one binade below each chunk maximum)."""
    z = rng.standard_normal(V).astype(np.float32) * 3
    if kind == 1:  # every logit negative: no chunk is counted, the window pass decides
        z -= 30
    elif kind == 2:  # one chunk of zeros, -0 and denormals: not counted, and far below the row's top
        z[8192:16384] = rng.choice(np.array([0.0, -0.0, 1e-39, 5e-39], dtype=np.float32), 8192)
    elif kind == 3:  # a tiny positive maximum: its window would reach +0
        z = rng.standard_normal(V).astype(np.float32) - 5
        z[rng.choice(V, 4, replace=False)] = np.array([1e-39, 2e-39, 3e-39, 4e-39], dtype=np.float32)
    elif kind == 4:  # a staircase of 300 keys below 8.0, three copies each, over a negative floor
        z = rng.standard_normal(V).astype(np.float32) - 10
        steps = W.bf16_to_f32(np.uint16(0x4100) - np.arange(300, dtype=np.uint16))
        z[rng.choice(V, 900, replace=False)] = np.repeat(steps, 3)
    elif kind == 5:  # peaked: three large logits over a N(0, 1) floor
        z = rng.standard_normal(V).astype(np.float32)
        z[rng.choice(V, 3, replace=False)] = np.array([14.0, 13.5, 13.0], dtype=np.float32)
    return z


def test_row_pass_counts_and_their_fallbacks():
    """Truncating bf16 calls count, in the row pass, the keys of the binade below each chunk's
    maximum, and cut from those counts when the cut lies inside that binade.  Rows here put the cut
    just inside and just outside it (a staircase of keys: top-k 382 ends on the 128th key, 385 on the
    129th), make a nucleus end inside it (a peaked row with top-p alone) or beyond it, and give
    chunks that cannot be counted (a maximum <= 0, or one whose binade would reach +0), alone or
    next to counted ones."""
    rng = np.random.default_rng(79)
    B, V, K = 48, 3 * 8192 + 1000, 2
    kinds = np.arange(B) % 6
    cu = W.offsets_from_depths(np.full(B, K))
    n_d = B * K
    tgt = np.empty((n_d + B, V), dtype=np.float32)
    drf = np.empty((n_d, V), dtype=np.float32)
    for i in range(B):
        for j in range(K + 1):
            tgt[cu[i] + i + j] = _counted_row(kinds[i], V, rng)
        for j in range(K):  # the target row with a tenth of its logits moved: drafts are often accepted
            d = tgt[cu[i] + i + j].copy()
            moved = rng.random(V) < 0.1
            d[moved] += rng.standard_normal(int(moved.sum())).astype(np.float32)
            drf[cu[i] + j] = d
    b = W.Batch(name="row_pass_counts", V=V, dtype="bf16", temperature=0.8, seed=13, target=W.bf16_bits(tgt),
                draft=W.bf16_bits(drf), tokens=np.zeros(n_d, dtype=np.int32), cu=cu)
    choices = {0: ([50, 200, 0], [900, 1000, 950]), 1: ([50, 0], [900]), 2: ([50, 0], [900, 950]),
               3: ([5, 50], [900, 1000]), 4: ([382, 384, 385, 386, 900], [1000, 990, 900]),
               5: ([0], [500, 900, 990])}
    nth = np.arange(B) // 6  # each kind's requests cycle through its profiles
    top_k = np.array([choices[k][0][n % len(choices[k][0])] for k, n in zip(kinds, nth)], dtype=np.int32)
    milli = np.array([choices[k][1][n % len(choices[k][1])] for k, n in zip(kinds, nth)], dtype=np.int32)
    b.tokens = drafter_tokens(b, top_k, milli, rng)
    acc, out, got, ref = check(b, top_k, milli)
    assert (acc >= 0).all()


def test_wide_rows_span_several_batches_of_chunks():
    """bf16 rows of 74 chunks (V = 600,000): the count kernel sums and scans chunk counts in batches
    of 64 chunks, and the full cut kernel's window pass has no per-chunk window counts (more than 32
    chunks), so its rows take the chunk pass.  Top-k values put cuts inside and below the counted
    binade."""
    rng = np.random.default_rng(83)
    B, V = 6, 600000
    depths = np.array([2, 1, 0, 2, 1, 2])
    cu = W.offsets_from_depths(depths)
    n_d = int(cu[-1])
    tgt = (rng.standard_normal((n_d + B, V)) * 3).astype(np.float32)
    t_of_d = np.concatenate([np.arange(cu[i], cu[i + 1]) + i for i in range(B)])
    drf = (tgt[t_of_d] + rng.standard_normal((n_d, V)) * 0.7).astype(np.float32)
    b = W.Batch(name="wide", V=V, dtype="bf16", temperature=1.0, seed=31, target=W.bf16_bits(tgt),
                draft=W.bf16_bits(drf), tokens=np.zeros(n_d, dtype=np.int32), cu=cu)
    top_k = np.array([50, 0, 300, 5000, 1, 0], dtype=np.int32)
    milli = np.array([900, 950, 1000, 990, 1000, 500], dtype=np.int32)
    b.tokens = drafter_tokens(b, top_k, milli, rng)
    check(b, top_k, milli)


def test_truncated_repeat_launches_are_deterministic():
    """The cuts rest on integer counts and fixed-point masses, and every reduction has a fixed
    order, so repeated calls give bit-identical outputs, kept counts and truncated LSEs: rows that
    the count kernel settles and rows it leaves to the full cut kernel alike."""
    rng = np.random.default_rng(89)
    B, V, K = 24, 3 * 8192 + 1000, 2
    kinds = np.arange(B) % 6
    cu = W.offsets_from_depths(np.full(B, K))
    n_d = B * K
    tgt = np.stack([_counted_row(kinds[r // (K + 1)], V, rng) for r in range(n_d + B)])
    drf = np.stack([_counted_row(kinds[d // K], V, rng) for d in range(n_d)])
    b = W.Batch(name="repeat_cuts", V=V, dtype="bf16", temperature=0.8, seed=17, target=W.bf16_bits(tgt),
                draft=W.bf16_bits(drf), tokens=np.zeros(n_d, dtype=np.int32), cu=cu)
    top_k = np.array([[50, 0, 50, 5, 385, 0][k] for k in kinds], dtype=np.int32)
    milli = np.array([[900, 900, 950, 1000, 990, 900][k] for k in kinds], dtype=np.int32)
    b.tokens = drafter_tokens(b, top_k, milli, rng)
    ins = (to_device(b.target, b.dtype), to_device(b.draft, b.dtype), torch.from_numpy(b.tokens).to(DEV),
           torch.from_numpy(b.cu).to(DEV))
    kw = {"top_k": torch.from_numpy(top_k).to(DEV), "top_p_milli": torch.from_numpy(milli).to(DEV)}
    diag = ("kept_tokens", "target_lse", "ratio")
    runs = []
    for _ in range(12):
        acc, out, extra = sdv.verify_ex(*ins, b.temperature, b.seed, diag=diag, **kw)
        torch.cuda.synchronize()
        runs.append((acc.cpu().numpy(), out.cpu().numpy(), {k: v.cpu().numpy() for k, v in extra.items()}))
    for acc, out, extra in runs[1:]:
        assert np.array_equal(acc, runs[0][0]) and np.array_equal(out, runs[0][1])
        for k in diag:
            assert np.array_equal(extra[k], runs[0][2][k], equal_nan=True), k
