"""Statistical exactness of the HIP path under top-k / top-p (SDCP, section "Session Contract":
temperature, then top-k, then top-p).

One fixed (target, draft) row pair per case, B = 4096 requests of depth 3, fresh draft tokens per
call drawn from the truncated draft distribution.  Two things are checked on the GPU's own verdicts:
  * every call equals the oracle's verdicts on the same inputs, up to counted near-ties;
  * the histograms of the accepted length and of the emitted token at each reached position follow
    the exact law of a round over the truncated rows (brute-force enumeration, oracle/exact.py, over
    the rows the per-token definition of filter_pins.py truncates): speculative sampling stays
    lossless for the truncated target distribution.
fp32 rows take the kernel's radix selection, bf16 rows its window of keys below the maximum.
"""
import numpy as np
import pytest
import torch

import filter_pins as F
import lossless_draft_verification_online_amd as sdv
import workloads as W
from gpu_helpers import DEV, log
from oracle import exact, oracle
from oracle.compare import compare_verdicts
from test_oracle_sampling import _pvalues

pytestmark = pytest.mark.gpu

K, B, T = 3, 4096, 0.9
N_CALLS = 100


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype,V,top_k,milli", [("fp32", 8, 5, 1000), ("fp32", 8, 0, 800), ("bf16", 16, 6, 900),
                                                 ("bf16", 16, 0, 700)])
def test_truncated_rounds_follow_the_exact_law(dtype, V, top_k, milli):
    rng = np.random.default_rng([V, top_k, milli])
    zt = (rng.standard_normal(V) * 1.5).astype(np.float32)
    zd = (zt + rng.standard_normal(V) * 0.8).astype(np.float32)
    if dtype == "bf16":  # the stored values are what both sides read
        zt, zd = W.bf16_to_f32(W.bf16_bits(zt)), W.bf16_to_f32(W.bf16_bits(zd))
    p = F.truncated_softmax(zt, T, top_k, milli)
    q = F.truncated_softmax(zd, T, top_k, milli)
    law = exact.round_distribution(np.stack([p] * (K + 1)), np.stack([q] * K), grid=True)
    store = (lambda a: W.bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    target = np.ascontiguousarray(np.broadcast_to(store(zt), (B * (K + 1), V)))
    draft = np.ascontiguousarray(np.broadcast_to(store(zd), (B * K, V)))
    tdev = (torch.from_numpy(target.view(np.int16)).to(DEV).view(torch.bfloat16) if dtype == "bf16"
            else torch.from_numpy(target).to(DEV))
    ddev = (torch.from_numpy(draft.view(np.int16)).to(DEV).view(torch.bfloat16) if dtype == "bf16"
            else torch.from_numpy(draft).to(DEV))
    cu = W.offsets_from_depths(np.full(B, K))
    cu_dev = torch.from_numpy(cu).to(DEV)
    tk = np.full(B, top_k, dtype=np.int32)
    tp = np.full(B, milli, dtype=np.int32)
    tk_dev, tp_dev = torch.from_numpy(tk).to(DEV), torch.from_numpy(tp).to(DEV)
    with np.errstate(divide="ignore"):
        logq = np.log(q)
    pmf = np.zeros(K + 1, dtype=np.int64)
    reached = np.zeros((K + 1, V), dtype=np.int64)
    excused = 0
    for c in range(N_CALLS):
        g = -np.log(-np.log(np.random.default_rng([7, V, top_k, milli, c]).random((B * K, V))))
        tokens = np.argmax(logq[None, :] + g, axis=1).astype(np.int32)
        seed = (c << 20) | (V << 8) | top_k
        acc, out, _ = sdv.verify_ex(tdev, ddev, torch.from_numpy(tokens).to(DEV), cu_dev, T, seed, top_k=tk_dev,
                                    top_p_milli=tp_dev)
        torch.cuda.synchronize()
        acc, out = acc.cpu().numpy(), out.cpu().numpy()
        ref = oracle.verify(target, draft, tokens, cu, T, seed, diag=True, top_k=tk, top_p_milli=tp)
        cmp = compare_verdicts(acc, out, ref, cu, T)
        assert cmp["n_hard"] == 0, f"call {c}: {cmp['hard'][:5]}"
        excused += cmp["n_excused"]
        assert (acc >= 0).all()
        pmf += np.bincount(acc, minlength=K + 1)
        slots = out.reshape(B, K + 1)
        for j in range(K + 1):
            reached[j] += np.bincount(slots[acc >= j, j], minlength=V)
    # tokens the truncated target drops are never emitted
    assert (reached[:, p == 0] == 0).all()
    keep = [j for j in range(K + 1) if law["token_reached"][j].sum() > 0]
    pv = _pvalues(pmf, reached[keep], {"pmf_accepted": law["pmf_accepted"],
                                       "token_reached": law["token_reached"][keep]})
    log(f"  {dtype} V={V} top_k={top_k} top_p={milli}/1000: {pmf.sum()} trials, kept {int((p > 0).sum())} / "
        f"{int((q > 0).sum())}, excuses {excused}, min p-value {min(pv):.3g}")
    assert min(pv) * len(pv) > 1e-5, pv
