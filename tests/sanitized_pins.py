"""Runs the oracle's pins and the SDCP HMAC check against builds made with AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).  Started by test_sanitizers.py in a child process whose
LD_PRELOAD names the sanitizer runtime, since the Python interpreter itself is not instrumented.

usage: sanitized_pins.py ORACLE_SO SDCP_SO
"""
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(HERE), HERE]

import numpy as np  # noqa: E402

import test_oracle_mutations as M  # noqa: E402
from oracle import sdcp  # noqa: E402
from workloads import offsets_from_depths  # noqa: E402


def oracle_pins(lib_path):
    for check in (M._pin_lse, M._pin_greedy_tie, M._pin_profiles, M._pin_stops, M._pin_qrows, M._pin_filters,
                  M._pin_keying, M._pin_tree, M._pin_monte_carlo):
        assert check(lib_path), check.__name__
        print(f"pin ok: {check.__name__}", flush=True)


def sdcp_check(lib_path):
    """The host HMAC-SHA-256 uniforms (sdv_sdcp_uniforms, built alone) against Python's hmac, on
    ragged batches including depth 0 and 64 and the extreme seeds and rounds."""
    lib = ctypes.CDLL(lib_path)
    lib.sdv_sdcp_uniforms.restype = ctypes.c_int
    lib.sdv_sdcp_uniforms.argtypes = [ctypes.c_int32] + [ctypes.c_void_p] * 6
    for seed in range(3):
        rng = np.random.default_rng(seed)
        depths = rng.integers(0, 9, size=40)
        depths[:2] = (0, 64)
        cu = offsets_from_depths(depths)
        B = cu.shape[0] - 1
        seeds = rng.integers(0, 2**63, size=B, dtype=np.int64).astype(np.uint64)
        seeds[:2] = (0, 2**64 - 1)
        sessions = rng.integers(0, 256, size=(B, 16), dtype=np.uint8)
        rounds = rng.integers(0, 2**32, size=B, dtype=np.uint64).astype(np.uint32)
        rounds[:2] = (0, 2**32 - 1)
        r = np.zeros(int(cu[-1]), dtype=np.float64)
        u = np.zeros(int(cu[-1]) + B, dtype=np.float64)
        rc = lib.sdv_sdcp_uniforms(B, cu.ctypes.data, seeds.ctypes.data, sessions.ctypes.data, rounds.ctypes.data,
                                   r.ctypes.data, u.ctypes.data)
        assert rc == 0, rc
        r_ref, u_ref = sdcp.batch_uniforms(cu, seeds, sessions, rounds)
        assert np.array_equal(r, r_ref) and np.array_equal(u, u_ref)
    # a malformed offsets array is refused, not read past
    bad = np.array([0, 3, 1], dtype=np.int32)
    r = np.zeros(4, dtype=np.float64)
    u = np.zeros(6, dtype=np.float64)
    z = np.zeros(2, dtype=np.uint64)
    s = np.zeros((2, 16), dtype=np.uint8)
    rd = np.zeros(2, dtype=np.uint32)
    assert lib.sdv_sdcp_uniforms(2, bad.ctypes.data, z.ctypes.data, s.ctypes.data, rd.ctypes.data, r.ctypes.data,
                                 u.ctypes.data) != 0
    print("sdcp ok", flush=True)


if __name__ == "__main__":
    oracle_pins(sys.argv[1])
    sdcp_check(sys.argv[2])
    print("sanitized pins ok", flush=True)
