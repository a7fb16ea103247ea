"""Lossless speculative-decoding verification on MI355X (gfx950).

Python face of libsdv.so (C ABI in include/sdv.h).  Tensors are torch tensors on the GPU; this
module only checks and marshals arguments, and every step of the verification runs in the HIP
kernels behind ``sdv_verify``.  Work goes on torch's current HIP stream.
"""
from __future__ import annotations

import contextlib
import ctypes

import torch

from . import _native
from ._native import (SDV_BF16, SDV_FP32, SDV_MAX_DEPTH, TERM_BAD, TERM_BONUS, TERM_GREEDY, TERM_NONE,
                      TERM_RESIDUAL, TERM_RESIDUAL_EMPTY, SdvError)

__all__ = ["verify", "verify_ex", "verify_tree", "commit", "repad", "workspace_bytes", "philox4x32_10", "philox_uniforms", "read_ceiling", "sdcp_uniforms", "abi_version", "SdvError", "SDV_MAX_DEPTH",
           "TERM_BAD", "TERM_BONUS", "TERM_GREEDY", "TERM_NONE", "TERM_RESIDUAL", "TERM_RESIDUAL_EMPTY", "library_path"]

_DTYPES = {torch.bfloat16: SDV_BF16, torch.float32: SDV_FP32}
_WORKSPACE: dict = {}


def library_path() -> str:
    return _native.lib()._name


def abi_version() -> int:
    return _native.lib().sdv_abi_version()


def workspace_bytes(B: int, n_draft_rows: int, V: int, dtype: torch.dtype) -> int:
    return int(_native.lib().sdv_workspace_bytes(B, n_draft_rows, V, _DTYPES[dtype]))


def _ptr(t):
    return None if t is None else t.data_ptr()


_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _launch_on(dev: torch.device):
    """(context, stream) for a launch on dev: the device guard (none when dev is already current)
    and the handle of dev's current stream.  The per-call entry points use it to keep their host
    cost small next to the kernels of a small batch."""
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    ctx = contextlib.nullcontext() if torch.cuda.current_device() == idx else torch.cuda.device(idx)
    stream = _RAW_STREAM(idx) if _RAW_STREAM is not None else torch.cuda.current_stream(idx).cuda_stream
    return ctx, stream


def _workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _WORKSPACE.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WORKSPACE[key] = ws
    return ws


def _profile_arrays(temperature, seed, B, dev):
    """Per-request profile tensors (temperature float32 [B], seed int64/uint64 [B] on the logits'
    device), or None for one scalar profile."""
    if not isinstance(temperature, torch.Tensor) and not isinstance(seed, torch.Tensor):
        return None
    if not (isinstance(temperature, torch.Tensor) and isinstance(seed, torch.Tensor)):
        raise ValueError("per-request profiles need both temperature and seed as [B] tensors")
    if temperature.dtype != torch.float32 or temperature.shape != (B,) or temperature.device != dev \
            or not temperature.is_contiguous():
        raise ValueError("temperature must be a contiguous float32 [B] tensor on the logits' device")
    if seed.dtype not in (torch.int64, torch.uint64) or seed.shape != (B,) or seed.device != dev \
            or not seed.is_contiguous():
        raise ValueError("seed must be a contiguous int64 or uint64 [B] tensor on the logits' device")
    return temperature, seed


def _check(target, draft, draft_tokens, offsets, temperature, draft_probs=None):
    if not target.is_cuda:
        raise ValueError("target logits must be on the GPU")
    if target.dtype not in _DTYPES:
        raise TypeError("logits must be bfloat16 or float32")
    if target.dim() != 2 or not target.is_contiguous():
        raise ValueError("target logits must be a contiguous [n_draft_rows + B, V] tensor")
    for name, t in (("draft_tokens", draft_tokens), ("offsets", offsets)):
        if t.dtype != torch.int32 or t.device != target.device or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 vector on the logits' device")
    if draft is not None:
        if draft.dtype != target.dtype or draft.device != target.device or not draft.is_contiguous():
            raise ValueError("draft logits must match the target's dtype and device and be contiguous")
        if draft.dim() != 2 or draft.shape[1] != target.shape[1] or draft.shape[0] != draft_tokens.shape[0]:
            raise ValueError("draft logits must be [n_draft_rows, V]")
    B = offsets.shape[0] - 1
    if target.shape[0] != draft_tokens.shape[0] + B:
        raise ValueError("target logits must have n_draft_rows + B rows")
    if draft_probs is not None:
        if draft_probs.dtype != torch.float32 or draft_probs.device != target.device or not draft_probs.is_contiguous() \
                or draft_probs.dim() != 2 or draft_probs.shape != (draft_tokens.shape[0], target.shape[1]):
            raise ValueError("draft_probs must be a contiguous float32 [n_draft_rows, V] tensor on the logits' device")
    needs_draft = isinstance(temperature, torch.Tensor) or temperature > 0
    if needs_draft and draft is None and draft_probs is None and draft_tokens.shape[0] > 0:
        raise ValueError("sampling (any temperature > 0, or per-request profiles) needs draft logits or draft_probs")


def _device_vector(t, dtype, n, dev, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != dev or t.dim() != 1 \
            or t.shape[0] != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} vector of {n} values on the logits' device")
    return t


def verify_ex(target: torch.Tensor, draft: torch.Tensor | None, draft_tokens: torch.Tensor, offsets: torch.Tensor,
              temperature, seed, *, out: tuple | None = None, workspace: torch.Tensor | None = None,
              diag: tuple[str, ...] = (), events: list | None = None, accept_uniform: torch.Tensor | None = None,
              draw_uniform: torch.Tensor | None = None, stop_offsets: torch.Tensor | None = None,
              stop_tokens: torch.Tensor | None = None, budget: torch.Tensor | None = None,
              draft_probs: torch.Tensor | None = None, top_k: torch.Tensor | None = None,
              top_p_milli: torch.Tensor | None = None, verdict_split: int = 0):
    """Run sdv_verify_ex; sdv_verify_profiled when temperature and seed are [B] device tensors (one
    sampling profile per request); sdv_verify_opts when the caller's uniforms (float64
    accept_uniform [n_draft_rows], draw_uniform [n_draft_rows + B]), stop lists (int32 CSR
    stop_offsets [B + 1], stop_tokens), a budget (int32 [B]) or draft_probs (float32
    [n_draft_rows, V], the draft distributions in place of draft logits) or the rest of the
    sampling profiles (int32 top_k [B], top_p_milli [B]) or verdict_split (workgroups per request
    in the verdict pass, 0: automatic) are given.  Returns (accepted_len,
    out_tokens, extra): extra holds the named diagnostic arrays (fields of sdv_diag, and with top-k /
    top-p "kept_tokens", int32 [n_draft_rows + B + n_draft_rows]) and "emitted_len" with stop lists
    or a budget.  ``events``: up to four torch.cuda.Event objects, recorded as sdv_diag.events
    describes.
    """
    _check(target, draft, draft_tokens, offsets, temperature, draft_probs)
    dev = target.device
    B = offsets.shape[0] - 1
    profile = _profile_arrays(temperature, seed, B, dev)
    n_d0 = draft_tokens.shape[0]
    accept_uniform = _device_vector(accept_uniform, torch.float64, n_d0, dev, "accept_uniform")
    draw_uniform = _device_vector(draw_uniform, torch.float64, n_d0 + B, dev, "draw_uniform")
    if (accept_uniform is None) != (draw_uniform is None):
        raise ValueError("accept_uniform and draw_uniform go together")
    stop_offsets = _device_vector(stop_offsets, torch.int32, B + 1, dev, "stop_offsets")
    if stop_offsets is not None:
        stop_tokens = stop_tokens if stop_tokens is not None else torch.empty(0, dtype=torch.int32, device=dev)
        stop_tokens = _device_vector(stop_tokens, torch.int32, stop_tokens.shape[0], dev, "stop_tokens")
    budget = _device_vector(budget, torch.int32, B, dev, "budget")
    top_k = _device_vector(top_k, torch.int32, B, dev, "top_k")
    top_p_milli = _device_vector(top_p_milli, torch.int32, B, dev, "top_p_milli")
    truncating = top_k is not None or top_p_milli is not None
    use_opts = (accept_uniform is not None or stop_offsets is not None or budget is not None or draft_probs is not None
                or truncating or verdict_split != 0)
    n_d = draft_tokens.shape[0]
    V = target.shape[1]
    dt = _DTYPES[target.dtype]
    if out is None:
        accepted_len = torch.empty(B, dtype=torch.int32, device=dev)
        out_tokens = torch.empty(n_d + B, dtype=torch.int32, device=dev)
    else:
        accepted_len, out_tokens = out
    # a caller's workspace is checked against the shape's need by the library itself
    ws = _workspace(int(_native.lib().sdv_workspace_bytes(B, n_d, V, dt)), dev) if workspace is None else workspace
    dvals = {}
    dg = None
    want_kept = "kept_tokens" in diag
    diag = tuple(name for name in diag if name != "kept_tokens")
    if diag or events:
        shapes = {"target_lse": (n_d + B, torch.float64), "draft_lse": (n_d, torch.float64),
                  "target_argmax": (n_d + B, torch.int32), "ratio": (n_d, torch.float64),
                  "accept_uniform": (n_d, torch.float32), "draw_uniform": (B, torch.float32),
                  "terminal_kind": (B, torch.int32), "target_logit": (n_d, torch.float32),
                  "draft_logit": (n_d, torch.float32), "terminal_mass": (B, torch.float64)}
        dg = _native.SdvDiag()
        for name in diag:
            n, t = shapes[name]
            fill = -9 if t == torch.int32 else float("nan")
            dvals[name] = torch.full((n,), fill, dtype=t, device=dev)
            setattr(dg, name, dvals[name].data_ptr())
        for k, ev in enumerate(events or []):
            if ev is not None:
                dg.events[k] = ev.cuda_event if hasattr(ev, "cuda_event") else int(ev)
    ctx, stream = _launch_on(dev)
    dg_ref = ctypes.byref(dg) if dg is not None else None
    with ctx:
        if use_opts:
            opt = _native.SdvOptions()
            if profile is not None:
                opt.temperature, opt.seed = _ptr(profile[0]), _ptr(profile[1])
            opt.accept_uniform, opt.draw_uniform = _ptr(accept_uniform), _ptr(draw_uniform)
            opt.draft_probs = _ptr(draft_probs)
            opt.verdict_split = int(verdict_split)
            if stop_offsets is not None:
                opt.stop_offsets, opt.stop_tokens = _ptr(stop_offsets), _ptr(stop_tokens)
                opt.n_stop_tokens = stop_tokens.shape[0]
            if stop_offsets is not None or budget is not None:
                opt.budget = _ptr(budget)
                dvals["emitted_len"] = torch.full((B,), -9, dtype=torch.int32, device=dev)
                opt.emitted_len = dvals["emitted_len"].data_ptr()
            if truncating:
                opt.top_k, opt.top_p_milli = _ptr(top_k), _ptr(top_p_milli)
                if want_kept:
                    dvals["kept_tokens"] = torch.full((2 * n_d + B,), -9, dtype=torch.int32, device=dev)
                    opt.kept_tokens = dvals["kept_tokens"].data_ptr()
            scalar_t = 0.0 if profile is not None else float(temperature)
            scalar_s = 0 if profile is not None else int(seed) & 0xFFFFFFFFFFFFFFFF
            rc = _native.lib().sdv_verify_opts(
                _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(offsets), B, n_d, V, dt, scalar_t, scalar_s,
                ctypes.byref(opt), _ptr(accepted_len), _ptr(out_tokens), _ptr(ws), ws.numel() * ws.element_size(),
                stream, dg_ref)
        elif profile is None:
            rc = _native.lib().sdv_verify_ex(
                _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(offsets), B, n_d, V, dt, float(temperature),
                int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(accepted_len), _ptr(out_tokens), _ptr(ws),
                ws.numel() * ws.element_size(), stream, dg_ref)
        else:
            rc = _native.lib().sdv_verify_profiled(
                _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(offsets), B, n_d, V, dt, _ptr(profile[0]),
                _ptr(profile[1]), _ptr(accepted_len), _ptr(out_tokens), _ptr(ws), ws.numel() * ws.element_size(),
                stream, dg_ref)
    if rc != 0:
        raise SdvError(rc, "sdv_verify_opts" if use_opts else
                       ("sdv_verify_profiled" if profile is not None else "sdv_verify_ex"))
    return accepted_len, out_tokens, dvals


def verify_tree(target: torch.Tensor, draft: torch.Tensor | None, draft_tokens: torch.Tensor, parents: torch.Tensor,
                offsets: torch.Tensor, temperature: float, seed: int, *, draft_row: torch.Tensor | None = None,
                out: tuple | None = None, workspace: torch.Tensor | None = None, diag: tuple[str, ...] = (),
                events: list | None = None):
    """sdv_verify_tree: token trees (int32 parents [n_nodes], each node's parent within its request,
    -1 for the root; target rows cu[i] + i at the root and cu[i] + i + n + 1 after node n; the logits
    node n was drawn from: draft row draft_row[cu[i] + n] (int32 [n_nodes]; siblings may share a
    row), or row cu[i] + n without draft_row).  Returns (accepted_len [B], out_tokens
    [n_nodes + B], accepted_nodes [n_nodes], extra) with the named sdv_diag arrays in extra; ``out``
    may hold those three output tensors."""
    _check(target, None, draft_tokens, offsets, 0.0, None)
    dev = target.device
    B = offsets.shape[0] - 1
    n = draft_tokens.shape[0]
    _device_vector(parents, torch.int32, n, dev, "parents")
    _device_vector(draft_row, torch.int32, n, dev, "draft_row")
    n_dr = n if draft_row is None else (draft.shape[0] if draft is not None else 0)
    if draft is not None:
        if draft.dtype != target.dtype or draft.device != dev or not draft.is_contiguous() or draft.dim() != 2 \
                or draft.shape[1] != target.shape[1] or draft.shape[0] != n_dr:
            raise ValueError("draft logits must be a contiguous [n_draft_rows, V] tensor like the target's")
    elif temperature > 0 and n_dr > 0:
        raise ValueError("temperature > 0 needs the draft logits")
    V = target.shape[1]
    dt = _DTYPES[target.dtype]
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(n + B, dtype=torch.int32, device=dev),
               torch.empty(n, dtype=torch.int32, device=dev))
    accepted_len, out_tokens, accepted_nodes = out
    need = int(_native.lib().sdv_workspace_bytes(B, n, V, dt))
    ws = _workspace(need, dev) if workspace is None else workspace
    shapes = {"target_lse": (n + B, torch.float64), "draft_lse": (n, torch.float64),
              "target_argmax": (n + B, torch.int32), "ratio": (n, torch.float64),
              "accept_uniform": (n, torch.float32), "draw_uniform": (B, torch.float32),
              "terminal_kind": (B, torch.int32), "target_logit": (n, torch.float32),
              "draft_logit": (n, torch.float32), "terminal_mass": (B, torch.float64)}
    dvals = {}
    dg = None
    if diag or events:
        dg = _native.SdvDiag()
        for name in diag:
            m, t = shapes[name]
            dvals[name] = torch.full((m,), -9 if t == torch.int32 else float("nan"), dtype=t, device=dev)
            setattr(dg, name, dvals[name].data_ptr())
        for k, ev in enumerate(events or []):
            if ev is not None:
                dg.events[k] = ev.cuda_event if hasattr(ev, "cuda_event") else int(ev)
    ctx, stream = _launch_on(dev)
    with ctx:
        rc = _native.lib().sdv_verify_tree(
            _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(parents), _ptr(draft_row), _ptr(offsets), B, n, n_dr, V, dt,
            float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(accepted_len), _ptr(accepted_nodes),
            _ptr(out_tokens), _ptr(ws), ws.numel() * ws.element_size(), stream,
            ctypes.byref(dg) if dg is not None else None)
    if rc != 0:
        raise SdvError(rc, "sdv_verify_tree")
    return accepted_len, out_tokens, accepted_nodes, dvals


def sdcp_uniforms(offsets, seeds, sessions, rounds):
    """SDCP's HMAC-SHA-256 uniforms on the host (sdv_sdcp_uniforms): offsets (B + 1,) int32, seeds
    (B,) uint64, sessions (B, 16) uint8, rounds (B,) uint32.  Returns numpy float64 arrays
    (accept_uniform [n_draft_rows], draw_uniform [n_draft_rows + B]) for verify_ex."""
    import numpy as np
    cu = np.ascontiguousarray(offsets, dtype=np.int32)
    B = cu.shape[0] - 1
    seeds = np.ascontiguousarray(seeds, dtype=np.uint64).reshape(B)
    sessions = np.ascontiguousarray(sessions, dtype=np.uint8).reshape(B, 16)
    rounds = np.ascontiguousarray(rounds, dtype=np.uint32).reshape(B)
    r = np.zeros(int(cu[-1]), dtype=np.float64)
    u = np.zeros(int(cu[-1]) + B, dtype=np.float64)
    rc = _native.lib().sdv_sdcp_uniforms(B, cu.ctypes.data, seeds.ctypes.data, sessions.ctypes.data,
                                         rounds.ctypes.data, r.ctypes.data if r.size else None, u.ctypes.data)
    if rc != 0:
        raise SdvError(rc, "sdv_sdcp_uniforms")
    return r, u


def verify(target: torch.Tensor, draft: torch.Tensor | None, draft_tokens: torch.Tensor, offsets: torch.Tensor,
           temperature, seed, *, out: tuple | None = None, workspace: torch.Tensor | None = None):
    """sdv_verify (or sdv_verify_profiled for [B] tensors of temperatures and seeds): (accepted_len [B]
    int32, out_tokens [n_draft_rows + B] int32), enqueued on the current stream."""
    a, o, _ = verify_ex(target, draft, draft_tokens, offsets, temperature, seed, out=out, workspace=workspace)
    return a, o


def philox4x32_10(counters: torch.Tensor, keys: torch.Tensor) -> torch.Tensor:
    """Raw device Philox4x32-10 blocks: counters [n, 4] and keys [n, 2] (int32 views of uint32 words)."""
    n = counters.shape[0]
    out = torch.empty((n, 4), dtype=torch.int32, device=counters.device)
    with torch.cuda.device(counters.device):
        rc = _native.lib().sdv_philox4x32_10(_ptr(counters), _ptr(keys), n, _ptr(out),
                                             torch.cuda.current_stream(counters.device).cuda_stream)
    if rc != 0:
        raise SdvError(rc, "sdv_philox4x32_10")
    return out


def philox_uniforms(seed: int, B: int, P: int, device="cuda") -> torch.Tensor:
    """The verifier's Philox blocks (sdv_philox_uniforms): int32 [B, P, 4] views of the uint32 words of
    the block of (request i, position j), counter (j, i, 0, 0), key = seed."""
    out = torch.empty((B, P, 4), dtype=torch.int32, device=device)
    with torch.cuda.device(out.device):
        rc = _native.lib().sdv_philox_uniforms(int(seed) & 0xFFFFFFFFFFFFFFFF, B, P, _ptr(out),
                                               torch.cuda.current_stream(out.device).cuda_stream)
    if rc != 0:
        raise SdvError(rc, "sdv_philox_uniforms")
    return out


READ_CHUNK_BYTES = 16384


def read_ceiling(src: torch.Tensor, out: torch.Tensor | None = None, shape: int = 0) -> torch.Tensor:
    """Reads with no arithmetic over a contiguous device buffer of whole 16 KiB chunks
    (sdv_read_yardstick; shape 0: the row pass's loads): returns the xor of each chunk's 32-bit words
    (int32 view), one per chunk."""
    nbytes = src.numel() * src.element_size()
    if not src.is_contiguous() or nbytes % READ_CHUNK_BYTES:
        raise ValueError("read_ceiling needs a contiguous buffer of whole 16 KiB chunks")
    n = nbytes // READ_CHUNK_BYTES
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=src.device)
    with torch.cuda.device(src.device):
        rc = _native.lib().sdv_read_yardstick(_ptr(src), n, int(shape), _ptr(out),
                                              torch.cuda.current_stream(src.device).cuda_stream)
    if rc != 0:
        raise SdvError(rc, "sdv_read_yardstick")
    return out


def commit(offsets: torch.Tensor, accepted_len: torch.Tensor, out_tokens: torch.Tensor, prefix_len: torch.Tensor,
           emitted_len: torch.Tensor | None = None) -> dict:
    """sdv_commit: the emitted tokens of a verified batch packed per request at contiguous logical
    positions, with each request's new lengths.  Returns device tensors offsets [B + 1],
    tokens / positions [n_draft_rows + B] (the first offsets[B] are used), lengths [B, 3]
    (L_out, L_target, L_draft), next_token [B], next_position [B]."""
    dev = offsets.device
    B = offsets.shape[0] - 1
    n_d = out_tokens.shape[0] - B
    for name, t, n in (("offsets", offsets, B + 1), ("accepted_len", accepted_len, B),
                       ("out_tokens", out_tokens, n_d + B), ("prefix_len", prefix_len, B)):
        _device_vector(t, torch.int32, n, dev, name)
    _device_vector(emitted_len, torch.int32, B, dev, "emitted_len")
    res = {"offsets": torch.empty(B + 1, dtype=torch.int32, device=dev),
           "tokens": torch.full((n_d + B,), -1, dtype=torch.int32, device=dev),
           "positions": torch.full((n_d + B,), -1, dtype=torch.int32, device=dev),
           "lengths": torch.empty((B, 3), dtype=torch.int32, device=dev),
           "next_token": torch.empty(B, dtype=torch.int32, device=dev),
           "next_position": torch.empty(B, dtype=torch.int32, device=dev)}
    with torch.cuda.device(dev):
        rc = _native.lib().sdv_commit(
            B, n_d, _ptr(offsets), _ptr(accepted_len), _ptr(emitted_len), _ptr(out_tokens), _ptr(prefix_len),
            _ptr(res["offsets"]), _ptr(res["tokens"]), _ptr(res["positions"]), _ptr(res["lengths"]),
            _ptr(res["next_token"]), _ptr(res["next_position"]), torch.cuda.current_stream(dev).cuda_stream)
    if rc != 0:
        raise SdvError(rc, "sdv_commit")
    return res


def repad(offsets: torch.Tensor, accepted_len: torch.Tensor, out_tokens: torch.Tensor, prefix_offsets: torch.Tensor,
          prefix_tokens: torch.Tensor, width: int, pad_id: int = 0, left_pad: bool = True,
          emitted_len: torch.Tensor | None = None) -> dict:
    """sdv_repad: each request's prefix (CSR: prefix_offsets [B + 1], prefix_tokens) followed by its
    emitted tokens, as rows of a [B, width] batch at logical positions 0 .. L - 1.  Returns device
    tensors token_ids [B, width] int32 (pad_id in padding), position_ids [B, width] int32 (-1 in
    padding), mask [B, width] uint8, row_len [B] int32 (L; -1 for malformed prefix offsets)."""
    dev = offsets.device
    B = offsets.shape[0] - 1
    n_d = out_tokens.shape[0] - B
    for name, t, n in (("offsets", offsets, B + 1), ("accepted_len", accepted_len, B),
                       ("out_tokens", out_tokens, n_d + B), ("prefix_offsets", prefix_offsets, B + 1)):
        _device_vector(t, torch.int32, n, dev, name)
    _device_vector(emitted_len, torch.int32, B, dev, "emitted_len")
    n_p = prefix_tokens.numel()
    _device_vector(prefix_tokens, torch.int32, n_p, dev, "prefix_tokens")
    res = {"token_ids": torch.empty((B, width), dtype=torch.int32, device=dev),
           "position_ids": torch.empty((B, width), dtype=torch.int32, device=dev),
           "mask": torch.empty((B, width), dtype=torch.uint8, device=dev),
           "row_len": torch.empty(B, dtype=torch.int32, device=dev)}
    with torch.cuda.device(dev):
        rc = _native.lib().sdv_repad(
            B, n_d, _ptr(offsets), _ptr(accepted_len), _ptr(emitted_len), _ptr(out_tokens), _ptr(prefix_offsets),
            _ptr(prefix_tokens) if n_p else None, n_p, int(width), int(pad_id), int(bool(left_pad)),
            _ptr(res["token_ids"]), _ptr(res["position_ids"]), _ptr(res["mask"]), _ptr(res["row_len"]),
            torch.cuda.current_stream(dev).cuda_stream)
    if rc != 0:
        raise SdvError(rc, "sdv_repad")
    return res
