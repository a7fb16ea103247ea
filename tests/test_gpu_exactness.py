"""Statistical exactness of the HIP path on the exactness workload (B=4096, K=3, V=8, fp32, one fixed
row pair per case, fresh draft tokens per call; 245 calls ~ 10^6 trials per case).

Two things are checked on the GPU's own verdicts:
  * every call equals the oracle's verdicts on the same inputs (same Philox uniforms), up to counted
    first divergences at decisions the oracle took within 1e-6 of its threshold;
  * the GPU's histograms of the accepted length and of the emitted token at each reached position
    follow the exact law of the method (brute-force enumeration, oracle/exact.py), and the mean
    accepted length is within 5 sigma of alpha (1 - alpha^K) / (1 - alpha) ("M7.8 - Speculative
    Serving", section 0x02; losslessness: SDCP Rule 2, "SOTA-227", "Why it is free rather than a
    trade").
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, log, run_gpu, run_oracle
from oracle import exact
from oracle.compare import compare_verdicts
from test_oracle_sampling import _pvalues
from workloads import exactness_batch, exactness_case

pytestmark = pytest.mark.gpu

N_CALLS = 245
K, V, B = 3, 8, 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("case", range(8))
def test_gpu_monte_carlo_matches_exact_law_and_oracle(case):
    zt, zd = exactness_case(case)
    p = exact.softmax(zt, 1.0)
    q = exact.softmax(zd, 1.0)
    law = exact.round_distribution(np.stack([p] * (K + 1)), np.stack([q] * K), grid=True)
    pmf = np.zeros(K + 1, dtype=np.int64)
    reached = np.zeros((K + 1, V), dtype=np.int64)
    t = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(zt, (B * (K + 1), V)))).to(DEV)
    d = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(zd, (B * K, V)))).to(DEV)
    excused = 0
    for c in range(N_CALLS):
        b = exactness_batch(case, c, rows=(zt, zd))
        ins = (t, d, torch.from_numpy(b.tokens).to(DEV), torch.from_numpy(b.cu).to(DEV))
        acc, out, _ = run_gpu(b, dev_inputs=ins)
        cmp = compare_verdicts(acc, out, run_oracle(b), b.cu, b.temperature)
        assert cmp["n_hard"] == 0, f"case {case} call {c}: {cmp['hard'][:5]}"
        excused += cmp["n_excused"]
        assert (acc >= 0).all()
        pmf += np.bincount(acc, minlength=K + 1)
        slots = out.reshape(B, K + 1)
        for j in range(K + 1):
            reached[j] += np.bincount(slots[acc >= j, j], minlength=V)
    pv = _pvalues(pmf, reached, law)
    log(f"  case {case}: {pmf.sum()} trials, near-tie excuses {excused}, min p-value {min(pv):.3g}")
    assert min(pv) * len(pv) > 1e-5, pv
    alpha = exact.acceptance_rate(p, q)
    n = pmf.sum()
    mean_a = (np.arange(K + 1) @ pmf) / n
    ea = alpha * (1 - alpha**K) / (1 - alpha)
    var_a = (np.arange(K + 1) ** 2) @ law["pmf_accepted"] - (np.arange(K + 1) @ law["pmf_accepted"]) ** 2
    assert abs(mean_a - ea) < 5 * np.sqrt(var_a / n)
