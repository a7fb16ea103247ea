"""sdv_verify_noalloc (the entry point for callers that cannot allocate) against sdv_verify.

Both run the same kernels; the no-alloc call keeps its workspace in the library's static device
array.  Outputs must be identical to sdv_verify's on the same inputs, on two calls in a row (the
second with a smaller batch, so the array holds the first call's leftovers), for a sampling and a
greedy batch; a batch beyond the array's size is refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, log, upload
from lossless_draft_verification_online_amd import _native

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _run(lib, b, noalloc):
    t, d, x, cu = upload(b)
    dt = _native.SDV_BF16 if b.dtype == "bf16" else _native.SDV_FP32
    acc = torch.full((b.B,), -9, dtype=torch.int32, device=DEV)
    out = torch.full((b.n_draft_rows + b.B,), -9, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    with torch.cuda.device(DEV):
        if noalloc:
            rc = lib.sdv_verify_noalloc(_ptr(t), _ptr(d), _ptr(x), _ptr(cu), b.B, b.n_draft_rows, b.V, dt,
                                        b.temperature, b.seed, _ptr(acc), _ptr(out), stream)
        else:
            need = lib.sdv_workspace_bytes(b.B, b.n_draft_rows, b.V, dt)
            ws = torch.empty(need, dtype=torch.uint8, device=DEV)
            rc = lib.sdv_verify(_ptr(t), _ptr(d), _ptr(x), _ptr(cu), b.B, b.n_draft_rows, b.V, dt, b.temperature,
                                b.seed, _ptr(acc), _ptr(out), _ptr(ws), need, stream)
    assert rc == 0, lib.sdv_status_string(rc)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def test_noalloc_matches_sdv_verify_on_two_calls():
    lib = _native.lib()
    rng = np.random.default_rng(2024)
    first = W.make_random("noalloc_first", rng.integers(0, 9, size=96), 128256, "bf16", 1.0, 3.0,
                          rng.uniform(0.5, 3.0, size=96), data_seed=91, verify_seed=0x1234)
    second = W.make_random("noalloc_second", rng.integers(0, 5, size=5), 1000, "fp32", 0.7, 2.0, 1.0,
                           data_seed=92, verify_seed=0x5678)
    greedy = W.make_random("noalloc_greedy", rng.integers(0, 7, size=33), 32000, "bf16", 0.0, 4.0, 1.0,
                           data_seed=93, verify_seed=0)
    for b in (first, second, greedy, second):
        dt = _native.SDV_BF16 if b.dtype == "bf16" else _native.SDV_FP32
        assert 0 < lib.sdv_noalloc_bytes(b.B, b.n_draft_rows, b.V, dt) <= _native_scratch_bytes()
        log(f"  noalloc {b.name}: B={b.B} V={b.V} T={b.temperature}")
        ref = _run(lib, b, noalloc=False)
        got = _run(lib, b, noalloc=True)
        assert np.array_equal(got[0], ref[0]), b.name
        assert np.array_equal(got[1], ref[1]), b.name
        assert (ref[0] >= 0).all()


def _native_scratch_bytes():
    return _native.SDV_NOALLOC_SCRATCH_BYTES


def test_noalloc_refuses_batches_beyond_its_scratch():
    lib = _native.lib()
    FAKE = 0x10000  # never dereferenced: the call is refused before any launch
    B, n_d, V = 4096, 60000, 128256
    assert lib.sdv_noalloc_bytes(B, n_d, V, 0) > _native_scratch_bytes()
    rc = lib.sdv_verify_noalloc(FAKE, FAKE, FAKE, FAKE, B, n_d, V, 0, 1.0, 1, FAKE, FAKE, None)
    assert rc == -3  # SDV_ERR_LIMIT
