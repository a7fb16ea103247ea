"""Pins for the oracle's Philox4x32-10 (Salmon et al., SC'11).

No known-answer vector appears in the pages.  The oracle's generator is pinned against rocRAND's
Philox4x32-10 engine (ROCm's own implementation, compiled here for the host and run), and its
words are checked for the uniformity and independence the verifier relies on.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROCRAND_HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


@pytest.fixture(scope="module")
def rocrand_probe(tmp_path_factory):
    if not os.path.exists(ROCRAND_HEADER) or shutil.which("g++") is None:
        pytest.skip("rocRAND headers or g++ not available")
    exe = str(tmp_path_factory.mktemp("probe") / "philox_probe")
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(HERE, "rocrand_philox_probe.cpp"), "-o", exe], check=True)
    return exe


def _rocrand_grid(exe, seed, n_req, n_pos, first_request=0):
    out = subprocess.run([exe, str(seed), str(first_request), str(n_req), str(n_pos)], check=True,
                         capture_output=True, text=True)
    words = np.array([[int(w, 16) for w in line.split()] for line in out.stdout.splitlines()], dtype=np.uint32)
    return words.reshape(n_req, n_pos, 4)


@pytest.mark.parametrize("seed", [0, 1, 0xDEADBEEF, 0x0123456789ABCDEF, 2**64 - 1, 20261202])
def test_philox_matches_rocrand(rocrand_probe, seed):
    ref = _rocrand_grid(rocrand_probe, seed, 40, 70)
    got = oracle.philox_grid(seed, 40, 70)
    assert np.array_equal(ref, got)


def test_philox_large_request_index(rocrand_probe):
    # high request ids exercise the second counter word fully
    seed = 0xA5A5A5A55A5A5A5A
    for req in (1 << 20, (1 << 30) - 1):
        ref = _rocrand_grid(rocrand_probe, seed, 1, 1, first_request=req)[0, 0]
        assert np.array_equal(ref, oracle.philox_block(seed, req, 0))


def test_philox_block_layout():
    # the block for (request i, position j) is Philox of counter (j, i, 0, 0) under key (seed lo, seed hi)
    seed = 0x1122334455667788
    for i, j in [(0, 0), (3, 5), (255, 8), (4095, 3)]:
        direct = oracle.philox4x32_10([j, i, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
        assert np.array_equal(direct, oracle.philox_block(seed, i, j))


def test_philox_words_uniform_and_independent():
    w = oracle.philox_grid(987654321, 4096, 256).reshape(-1, 4)  # 2^20 blocks
    for k in range(4):
        top = (w[:, k] >> 24).astype(np.int64)  # 256 bins on the top byte
        counts = np.bincount(top, minlength=256)
        assert stats.chisquare(counts).pvalue > 1e-6
    r = ((w[:, 0] >> 8) + 1) / 2.0**24
    u = (w[:, 1] >> 8) / 2.0**24
    assert r.min() > 0.0 and r.max() <= 1.0 and u.min() >= 0.0 and u.max() < 1.0
    assert stats.kstest(u, "uniform").pvalue > 1e-6
    # the two purposes (accept test, extra-token draw) must be uncorrelated
    assert abs(np.corrcoef(r, u)[0, 1]) < 5.0 / np.sqrt(r.size)
    # joint 16x16 histogram of (r, u) is flat
    joint = np.histogram2d(r, u, bins=16, range=[[0, 1], [0, 1]])[0].ravel()
    assert stats.chisquare(joint).pvalue > 1e-6
