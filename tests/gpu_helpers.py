"""Shared helpers for the GPU parity tests: upload a workload, run the HIP path through the C ABI
(via the package's ctypes binding), run the oracle on the same inputs, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import lossless_draft_verification_online_amd as sdv
from oracle import oracle
from oracle.compare import compare_verdicts

DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(a: np.ndarray | None, dtype: str):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_device_off_grid(a: np.ndarray | None, dtype: str, shift: int):
    """a on the device, `shift` elements into a fresh buffer (shift > 0: its base sits on an element
    boundary only, off the 16-byte grid)."""
    if a is None:
        return None
    t = to_device(a, dtype)
    if shift == 0:
        return t
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=DEV)
    view = flat[shift:shift + t.numel()].view(t.shape)
    view.copy_(t)
    assert view.data_ptr() % 16 != 0
    return view


def upload(b):
    return (to_device(b.target, b.dtype), to_device(b.draft, b.dtype),
            torch.from_numpy(b.tokens).to(DEV), torch.from_numpy(b.cu).to(DEV))


def profile_args(b, seed=None):
    """(temperature, seed) for the GPU call: scalars, or [B] device tensors for a profiled batch."""
    if b.temp_each is None:
        return b.temperature, (b.seed if seed is None else seed)
    return (torch.from_numpy(np.ascontiguousarray(b.temp_each, dtype=np.float32)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(b.seed_each, dtype=np.uint64).view(np.int64)).to(DEV))


def run_gpu(b, diag=(), seed=None, dev_inputs=None):
    t, d, x, cu = upload(b) if dev_inputs is None else dev_inputs
    temperature, sd = profile_args(b, seed)
    kw = {}
    if b.qrows is not None:
        kw["draft_probs"] = torch.from_numpy(b.qrows).to(DEV)
    acc, out, dg = sdv.verify_ex(t, d, x, cu, temperature, sd, diag=diag, **kw)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy(), {k: v.cpu().numpy() for k, v in dg.items()}


def run_oracle(b, seed=None):
    kw = {} if b.qrows is None else {"draft_probs": b.qrows}
    if b.temp_each is not None:
        return oracle.verify(b.target, b.draft, b.tokens, b.cu, b.temp_each.astype(np.float64), b.seed_each,
                             diag=True, **kw)
    return oracle.verify(b.target, b.draft, b.tokens, b.cu, b.temperature, b.seed if seed is None else seed,
                         diag=True, **kw)


def check_parity(b, seed=None, eps=1e-6, dev_inputs=None, diag=("terminal_kind",)):
    """GPU verdicts equal the oracle's, except first divergences at oracle margins below eps."""
    log(f"  parity {b.name}: B={b.B} n_draft_rows={b.n_draft_rows} V={b.V} {b.dtype} T={b.temperature}")
    acc, out, dg = run_gpu(b, diag=diag, seed=seed, dev_inputs=dev_inputs)
    ref = run_oracle(b, seed=seed)
    temperature = b.temp_each.astype(np.float64) if b.temp_each is not None else b.temperature
    cmp = compare_verdicts(acc, out, ref, b.cu, temperature, eps=eps)
    assert cmp["n_hard"] == 0, f"{b.name}: hard mismatches {cmp['hard'][:10]}"
    return acc, out, ref, cmp, dg
