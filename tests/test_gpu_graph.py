"""The verification captured in a HIP graph (torch.cuda.graph over the C-ABI calls) and replayed: every
replay, with other eager GPU work and synchronizations in between, gives the eager call's outputs.
The library records no memset and allocates nothing inside a call, so its launches capture as they
are; this is what bench.py --graph replays."""
import numpy as np
import pytest
import torch

import lossless_draft_verification_online_amd as sdv
import workloads as W
from gpu_helpers import DEV, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _replays_match(call, outs, other):
    """call(outs) enqueues the verification into the output tensors `outs`."""
    call(outs)
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(outs)
    for r in range(3):
        for o in outs:
            o.fill_(-5)
        other()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("V,dtype,truncate", [(4096, "fp32", False), (32000, "bf16", False), (32000, "bf16", True)])
def test_linear_verification_replays(V, dtype, truncate):
    rng = np.random.default_rng(V + truncate)
    b = W.make_random("graph", rng.integers(0, 9, size=32), V, dtype, 1.0, 2.5, 1.2, data_seed=V, verify_seed=3)
    t, d, x, cu = to_device(b.target, dtype), to_device(b.draft, dtype), _i32(b.tokens), _i32(b.cu)
    ws = torch.empty(sdv.workspace_bytes(b.B, b.n_draft_rows, V, t.dtype), dtype=torch.uint8, device=DEV)
    kw = {}
    if truncate:
        kw = {"top_k": _i32(np.full(b.B, 50)), "top_p_milli": _i32(np.full(b.B, 900))}
        x = _i32(np.argmax(b.draft_f32(), axis=1))  # the draft argmax: kept by every truncation
    outs = [torch.empty(b.B, dtype=torch.int32, device=DEV), torch.empty(b.n_draft_rows + b.B, dtype=torch.int32,
                                                                         device=DEV)]
    other_t = torch.randn_like(t.float()).to(t.dtype)

    def other():
        sdv.verify_ex(other_t, d, x, cu, 0.7, 99, workspace=ws, **kw)

    _replays_match(lambda o: sdv.verify_ex(t, d, x, cu, 1.0, 3, out=tuple(o), workspace=ws, **kw), outs, other)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_one_request_replays(T):
    """A batch of one small request (the single-launch path) captured and replayed."""
    b = W.make_random("graph_one", [4], 1000, "fp32", T, 2.0, 1.0, data_seed=11, verify_seed=12, keep_draft=True)
    t, d, x, cu = to_device(b.target, "fp32"), to_device(b.draft, "fp32"), _i32(b.tokens), _i32(b.cu)
    ws = torch.empty(sdv.workspace_bytes(b.B, b.n_draft_rows, b.V, t.dtype), dtype=torch.uint8, device=DEV)
    outs = [torch.empty(1, dtype=torch.int32, device=DEV), torch.empty(b.n_draft_rows + 1, dtype=torch.int32,
                                                                       device=DEV)]
    other_t = torch.randn_like(t)

    def other():
        sdv.verify_ex(other_t, d, x, cu, 0.7, 99, workspace=ws)

    _replays_match(lambda o: sdv.verify_ex(t, d, x, cu, T, 3, out=tuple(o), workspace=ws), outs, other)


def test_tree_verification_replays():
    rng = np.random.default_rng(5)
    b = W.make_tree("graph_tree", rng.integers(0, 20, size=24), "random", 32000, "bf16", 1.0, 2.5, 1.5, data_seed=6,
                    verify_seed=7, shared=True)
    t, d = to_device(b.target, b.dtype), to_device(b.draft, b.dtype)
    x, par, rows, cu = _i32(b.tokens), _i32(b.parents), _i32(b.draft_row), _i32(b.cu)
    ws = torch.empty(sdv.workspace_bytes(b.B, b.n_draft_rows, b.V, t.dtype), dtype=torch.uint8, device=DEV)
    outs = [torch.empty(b.B, dtype=torch.int32, device=DEV),
            torch.empty(b.n_draft_rows + b.B, dtype=torch.int32, device=DEV),
            torch.empty(b.n_draft_rows, dtype=torch.int32, device=DEV)]

    def other():
        torch.cuda.synchronize()
        (t.float() * 2).sum().item()

    _replays_match(lambda o: sdv.verify_tree(t, d, x, par, cu, 1.0, 7, draft_row=rows, out=tuple(o), workspace=ws),
                   outs, other)
