"""GPU parity of sdv_commit (post-verification unpad/append/repad, "M7.8 - Speculative Serving",
sections 0x03C, 0x03D and 0x09) against the plain reference in oracle/commit.py: integer work,
compared exactly."""
import numpy as np
import pytest
import torch

import lossless_draft_verification_online_amd as sdv
import workloads as W
from gpu_helpers import DEV, to_device
from oracle import commit as C
from oracle import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _compare(cu, acc, out, prefix, emitted=None):
    got = sdv.commit(_dev(cu), _dev(acc), _dev(out), _dev(prefix), None if emitted is None else _dev(emitted))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in got.items()}
    ref = C.commit(cu, acc, out, prefix, emitted_len=emitted)
    total = int(ref["offsets"][-1])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["tokens"][:total], ref["tokens"]) and np.array_equal(got["positions"][:total], ref["positions"])
    for k in ("lengths", "next_token", "next_position"):
        assert np.array_equal(got[k], ref[k]), k


def test_commit_after_gpu_verification_with_stops():
    rng = np.random.default_rng(1)
    b = W.make_random("commit", rng.integers(0, 9, size=200), 4099, "fp32", 1.0, 2.0, 1.0, data_seed=2, verify_seed=3)
    stops = [list(rng.choice(4099, size=2, replace=False)) + [int(b.tokens[b.cu[i]])] if b.cu[i + 1] > b.cu[i]
             and rng.random() < 0.3 else [] for i in range(b.B)]
    offs, toks = oracle.stop_csr(stops)
    budget = rng.integers(0, 12, size=b.B).astype(np.int32)
    acc, out, extra = sdv.verify_ex(to_device(b.target, b.dtype), to_device(b.draft, b.dtype), _dev(b.tokens),
                                    _dev(b.cu), 1.0, 3, stop_offsets=_dev(offs), stop_tokens=_dev(toks),
                                    budget=_dev(budget))
    torch.cuda.synchronize()
    prefix = rng.integers(0, 5000, size=b.B)
    _compare(b.cu, acc.cpu().numpy(), out.cpu().numpy(), prefix, extra["emitted_len"].cpu().numpy())
    _compare(b.cu, acc.cpu().numpy(), out.cpu().numpy(), prefix)  # without emitted counts: a + 1 each


@pytest.mark.parametrize("B", [1, 1023, 1024, 1025, 3000])
def test_commit_tiles_and_rejections(B):
    rng = np.random.default_rng(B)
    cu = W.offsets_from_depths(rng.integers(0, 9, size=B))
    K = np.diff(cu)
    acc = np.array([rng.integers(0, k + 1) if rng.random() > 0.05 else -1 for k in K], dtype=np.int32)
    out = rng.integers(0, 50000, size=int(cu[-1]) + B).astype(np.int32)
    emitted = np.array([rng.integers(-1, a + 3) for a in np.maximum(acc, 0)], dtype=np.int32)
    _compare(cu, acc, out, rng.integers(0, 10**6, size=B), emitted)


def test_malformed_offsets_emit_nothing_and_stay_in_bounds():
    cu = np.array([0, 5, 0, 5, 0, 5], dtype=np.int32)  # rises and falls: K = 5, -5, 5, -5, 5
    acc = np.array([5, 0, 5, 0, 5], dtype=np.int32)
    out = np.arange(10, dtype=np.int32)
    got = sdv.commit(_dev(cu), _dev(acc), _dev(out), _dev(np.zeros(5)))
    torch.cuda.synchronize()
    # requests 1 and 3 (negative depth) emit nothing; the others overlap, so the offsets run past the
    # 10-entry arrays: the counts are reported as they are, and no token is written beyond entry 9
    ref = C.commit(cu, acc, out, np.zeros(5))
    assert np.array_equal(got["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(got["tokens"].cpu().numpy(), ref["tokens"][:10])
    assert np.array_equal(got["lengths"].cpu().numpy(), ref["lengths"])


def _compare_repad(cu, acc, out, po, pt, width, pad_id, left, emitted=None):
    got = sdv.repad(_dev(cu), _dev(acc), _dev(out), _dev(po), _dev(pt), width, pad_id, left,
                    None if emitted is None else _dev(emitted))
    torch.cuda.synchronize()
    ref = C.repad(cu, acc, out, po, pt, width, pad_id, left, emitted_len=emitted)
    for k in ("token_ids", "position_ids", "mask", "row_len"):
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k
    return ref


def test_repad_after_gpu_verification_with_stops():
    """Section 0x03D's repad of a verified batch: prefix + emitted tokens per row, both padding
    sides, at the section's width (the longest row) and at a width the longest rows overflow."""
    rng = np.random.default_rng(21)
    b = W.make_random("repad", rng.integers(0, 9, size=150), 4099, "fp32", 1.0, 2.0, 1.0, data_seed=22, verify_seed=23)
    stops = [[int(b.tokens[b.cu[i]])] if b.cu[i + 1] > b.cu[i] and rng.random() < 0.3 else [] for i in range(b.B)]
    offs, toks = oracle.stop_csr(stops)
    budget = rng.integers(0, 12, size=b.B).astype(np.int32)
    acc, out, extra = sdv.verify_ex(to_device(b.target, b.dtype), to_device(b.draft, b.dtype), _dev(b.tokens),
                                    _dev(b.cu), 1.0, 23, stop_offsets=_dev(offs), stop_tokens=_dev(toks),
                                    budget=_dev(budget))
    torch.cuda.synchronize()
    acc, out, emitted = acc.cpu().numpy(), out.cpu().numpy(), extra["emitted_len"].cpu().numpy()
    plen = rng.integers(0, 40, size=b.B)
    po = np.concatenate([[0], np.cumsum(plen)])
    pt = rng.integers(0, 4099, size=int(po[-1]))
    width = int(np.max(plen + emitted))
    for w in (width, width - 2):
        for left in (True, False):
            ref = _compare_repad(b.cu, acc, out, po, pt, w, -5, left, emitted)
    assert (ref["row_len"] > width - 2).any()


@pytest.mark.parametrize("B,width", [(1, 7), (3000, 1000)])
def test_repad_grid_stride_and_malformed_prefixes(B, width):
    """3000 x 1000 cells exceed one pass of the grid (8192 workgroups of 256 threads), so cells are
    revisited by the stride loop; a few rows get decreasing or out-of-range prefix offsets."""
    rng = np.random.default_rng(B)
    cu = W.offsets_from_depths(rng.integers(0, 9, size=B))
    K = np.diff(cu)
    acc = np.array([rng.integers(0, k + 1) if rng.random() > 0.05 else -1 for k in K], dtype=np.int32)
    out = rng.integers(0, 50000, size=int(cu[-1]) + B).astype(np.int32)
    emitted = np.array([rng.integers(-1, a + 3) for a in np.maximum(acc, 0)], dtype=np.int32)
    po = np.concatenate([[0], np.cumsum(rng.integers(0, width, size=B))]).astype(np.int64)
    pt = rng.integers(0, 50000, size=int(po[-1]))
    if B > 2:
        po[B // 2] = po[B // 2 + 1] + 3  # row B/2 - 1 grows, row B/2 decreases
        po[B // 2 + 3] = po[-1] + 5  # beyond the prefix tokens: rows B/2 + 2 and B/2 + 3
        po[B // 2] = min(po[B // 2], po[-1])
    for left in (True, False):
        ref = _compare_repad(cu, acc, out, po, pt, width, 0, left, emitted)
    if B > 2:
        assert (ref["row_len"] == -1).sum() >= 2
