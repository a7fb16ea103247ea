"""The library's host-side SDCP uniforms (sdv_sdcp_uniforms: its own SHA-256 and HMAC) against
Python's standard hmac/hashlib ("Speculative Decoding Coordination Protocol (SDCP)", section
"Acceptance Rules", Rule 2).  Runs on the CPU: the function is host code."""
import numpy as np
import pytest
from scipy import stats

import lossless_draft_verification_online_amd as sdv
from lossless_draft_verification_online_amd import _native
from lossless_draft_verification_online_amd.build import is_stale
from oracle import sdcp
from workloads import offsets_from_depths


@pytest.fixture(scope="module", autouse=True)
def _built():
    if is_stale():
        pytest.fail("libsdv.so is missing or older than its sources; run __graft_entry__.build()")


def _batch(B, seed):
    rng = np.random.default_rng(seed)
    cu = offsets_from_depths(rng.integers(0, 9, size=B))
    seeds = rng.integers(0, 2**63, size=B, dtype=np.int64).astype(np.uint64) * np.uint64(2) + np.uint64(seed % 2)
    sessions = rng.integers(0, 256, size=(B, 16), dtype=np.uint8)
    rounds = rng.integers(0, 2**32, size=B, dtype=np.uint64).astype(np.uint32)
    return cu, seeds, sessions, rounds


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_library_matches_python_hmac(seed):
    cu, seeds, sessions, rounds = _batch(40, seed)
    r, u = sdv.sdcp_uniforms(cu, seeds, sessions, rounds)
    r_ref, u_ref = sdcp.batch_uniforms(cu, seeds, sessions, rounds)
    assert np.array_equal(r, r_ref) and np.array_equal(u, u_ref)


def test_edge_seeds_and_rounds():
    cu = offsets_from_depths([1, 0, 64])
    seeds = np.array([0, 2**64 - 1, 0x0102030405060708], dtype=np.uint64)
    sessions = np.array([[0] * 16, [255] * 16, list(range(16))], dtype=np.uint8)
    rounds = np.array([0, 2**32 - 1, 7], dtype=np.uint32)
    r, u = sdv.sdcp_uniforms(cu, seeds, sessions, rounds)
    r_ref, u_ref = sdcp.batch_uniforms(cu, seeds, sessions, rounds)
    assert np.array_equal(r, r_ref) and np.array_equal(u, u_ref)


def test_values_on_the_53_bit_grid_and_uniform():
    cu, seeds, sessions, rounds = _batch(2000, 9)
    r, u = sdv.sdcp_uniforms(cu, seeds, sessions, rounds)
    for x in (r, u):
        assert ((x >= 0) & (x < 1)).all()
        assert np.array_equal(x * 2.0**53, np.floor(x * 2.0**53))
    assert stats.kstest(np.concatenate([r, u]), "uniform").pvalue > 1e-4


def test_invalid_offsets_are_rejected():
    L = _native.lib()
    seeds = np.zeros(2, dtype=np.uint64)
    sessions = np.zeros((2, 16), dtype=np.uint8)
    rounds = np.zeros(2, dtype=np.uint32)
    r = np.zeros(8)
    u = np.zeros(8)
    for cu in ([0, 3, 2], [1, 2, 3], [0, 65, 66]):
        cu = np.array(cu, dtype=np.int32)
        assert L.sdv_sdcp_uniforms(2, cu.ctypes.data, seeds.ctypes.data, sessions.ctypes.data, rounds.ctypes.data,
                                   r.ctypes.data, u.ctypes.data) == -1
