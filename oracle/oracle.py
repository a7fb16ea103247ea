"""ctypes binding of the fp64 C oracle (``oracle/sdv_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this module.  It builds ``liboracle.so`` with gcc on first use if it is missing.

Semantics (each documented where the C source defines it):
  * Rule 1 (greedy) and Rule 2 (speculative sampling) of "Speculative Decoding Coordination
    Protocol (SDCP)", section "Acceptance Rules"; the accept test r <= p/q of "SOTA-227", section
    "What to do".
  * ragged batches: request i owns draft rows cu[i]..cu[i+1]-1 and target rows cu[i]+i..cu[i+1]+i
    ("M7.8 - Speculative Serving", section 0x00, its background on the serving unit: one extra
    target row per request beyond its K_i).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sdv_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

BF16, FP32 = 0, 1
TERM_GREEDY, TERM_BONUS, TERM_RESIDUAL, TERM_RESIDUAL_EMPTY, TERM_NONE, TERM_BAD = 0, 1, 2, 3, 4, -1


def build(out: str = LIBRARY, extra_flags: tuple[str, ...] = ()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, fp64, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", *extra_flags, SOURCE, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class _Options(ctypes.Structure):
    _fields_ = [
        ("temperature", ctypes.c_void_p),
        ("seed", ctypes.c_void_p),
        ("accept_uniform", ctypes.c_void_p),
        ("draw_uniform", ctypes.c_void_p),
        ("stop_offsets", ctypes.c_void_p),
        ("stop_tokens", ctypes.c_void_p),
        ("n_stop_tokens", ctypes.c_int64),
        ("budget", ctypes.c_void_p),
        ("emitted_len", ctypes.c_void_p),
        ("draft_probs", ctypes.c_void_p),
        ("top_k", ctypes.c_void_p),
        ("top_p_milli", ctypes.c_void_p),
        ("kept_tokens", ctypes.c_void_p),
    ]


class _Diag(ctypes.Structure):
    _fields_ = [
        ("target_lse", ctypes.c_void_p),
        ("draft_lse", ctypes.c_void_p),
        ("target_argmax", ctypes.c_void_p),
        ("ratio", ctypes.c_void_p),
        ("accept_margin", ctypes.c_void_p),
        ("cdf_margin", ctypes.c_void_p),
        ("resid_mass", ctypes.c_void_p),
        ("terminal_kind", ctypes.c_void_p),
        ("filter_margin", ctypes.c_void_p),
    ]


_LIBS: dict[str, ctypes.CDLL] = {}


def load(path: str = LIBRARY) -> ctypes.CDLL:
    if path in _LIBS:
        return _LIBS[path]
    if not os.path.exists(path) or (path == LIBRARY and os.path.getmtime(path) < os.path.getmtime(SOURCE)):
        build(path)
    lib = ctypes.CDLL(path)
    lib.oracle_verify.restype = ctypes.c_int
    lib.oracle_verify.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_uint64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Diag),
    ]
    lib.oracle_verify_opts.restype = ctypes.c_int
    lib.oracle_verify_opts.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_uint64,
        ctypes.POINTER(_Options), ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Diag),
    ]
    lib.oracle_verify_profiled.restype = ctypes.c_int
    lib.oracle_verify_profiled.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Diag),
    ]
    lib.oracle_verify_tree.restype = ctypes.c_int
    lib.oracle_verify_tree.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_uint64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Diag),
    ]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_philox_block.restype = None
    lib.oracle_philox_block.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    lib.oracle_philox_grid.restype = None
    lib.oracle_philox_grid.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.oracle_row_lse.restype = ctypes.c_double
    lib.oracle_row_lse.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_double]
    lib.oracle_row_argmax.restype = ctypes.c_int32
    lib.oracle_row_argmax.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32]
    lib.oracle_truncate_row.restype = ctypes.c_int32
    lib.oracle_truncate_row.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_int64,
        ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
    ]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    _LIBS[path] = lib
    return lib


def _ptr(a: np.ndarray | None) -> int | None:
    return None if a is None else a.ctypes.data


def _dtype_code(logits: np.ndarray) -> int:
    if logits.dtype == np.uint16:
        return BF16  # bf16 stored as its 16 raw bits
    if logits.dtype == np.float32:
        return FP32
    raise TypeError(f"logits must be uint16 (bf16 bits) or float32, got {logits.dtype}")


def stop_csr(stop_lists) -> tuple[np.ndarray, np.ndarray]:
    """Per-request stop-token lists as (offsets [B + 1], tokens) int32 arrays."""
    offs = np.concatenate([[0], np.cumsum([len(x) for x in stop_lists])]).astype(np.int32)
    toks = np.asarray([t for x in stop_lists for t in x], dtype=np.int32)
    return offs, toks


def verify(target: np.ndarray, draft: np.ndarray | None, draft_tokens: np.ndarray, cu: np.ndarray,
           temperature, seed, diag: bool = False, lib_path: str = LIBRARY, *, accept_uniform=None,
           draw_uniform=None, stop_lists=None, budget=None, draft_probs=None, top_k=None,
           top_p_milli=None) -> dict:
    """Run the oracle on one ragged batch.

    target: (n_draft_rows + B, V); draft: (n_draft_rows, V) or None when temperature == 0;
    draft_tokens: (n_draft_rows,) int32; cu: (B + 1,) int32 exclusive prefix sums of K_i.
    temperature and seed are scalars, or arrays of B values (one sampling profile per request).
    accept_uniform (n_draft_rows,) / draw_uniform (n_draft_rows + B,): the caller's uniforms in
    [0, 1), both or neither; stop_lists: B lists of stop tokens; budget: (B,) remaining outputs;
    draft_probs: (n_draft_rows, V) float32 draft distributions used in place of the draft logits;
    top_k / top_p_milli: (B,) the rest of each request's sampling profile (0 and 1000: no
    truncation).
    Returns accepted_len (B,), out_tokens (n_draft_rows + B,), emitted_len (B,) when stops or a
    budget are given, kept_tokens (n_draft_rows + B + n_draft_rows,) when top-k / top-p are given,
    and with ``diag`` the per-row LSEs, argmaxes, ratios, margins (filter_margin per row),
    residual masses and terminal kinds.
    """
    lib = load(lib_path)
    target = np.ascontiguousarray(target)
    dt = _dtype_code(target)
    if draft is not None:
        draft = np.ascontiguousarray(draft)
        if _dtype_code(draft) != dt:
            raise TypeError("target and draft must share a dtype")
    draft_tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    B = cu.shape[0] - 1
    n_d = draft_tokens.shape[0]
    V = target.shape[1]
    if target.shape[0] != n_d + B:
        raise ValueError("target must have n_draft_rows + B rows")
    acc = np.full(B, -7, dtype=np.int32)
    out = np.full(n_d + B, -7, dtype=np.int32)
    res: dict = {"accepted_len": acc, "out_tokens": out}
    dg_p = None
    if diag:
        n_t = n_d + B
        res.update(
            target_lse=np.full(n_t, np.nan), draft_lse=np.full(n_d, np.nan),
            target_argmax=np.full(n_t, -1, dtype=np.int32), ratio=np.full(n_d, np.nan),
            accept_margin=np.full(n_d, np.nan), cdf_margin=np.full(B, np.nan),
            resid_mass=np.full(B, np.nan), terminal_kind=np.full(B, -9, dtype=np.int32),
            filter_margin=np.full(n_t + n_d, np.inf),
        )
        dg = _Diag(*[_ptr(res[f]) for f, _ in _Diag._fields_])
        dg_p = ctypes.pointer(dg)
    extras = (accept_uniform is not None or draw_uniform is not None or stop_lists is not None or budget is not None
              or draft_probs is not None or top_k is not None or top_p_milli is not None)
    if extras:
        keep = []  # arrays the options point into stay alive for the call

        def arr(x, dtype, n):
            a = np.ascontiguousarray(np.asarray(x, dtype=dtype).reshape(n))
            keep.append(a)
            return _ptr(a)

        opt = _Options()
        if np.ndim(temperature) or np.ndim(seed):
            opt.temperature = arr(np.broadcast_to(np.asarray(temperature, dtype=np.float64), (B,)), np.float64, B)
            sd = np.asarray([int(x) & 0xFFFFFFFFFFFFFFFF for x in np.ravel(seed)], dtype=np.uint64) \
                if np.ndim(seed) else np.full(B, int(seed) & 0xFFFFFFFFFFFFFFFF, dtype=np.uint64)
            opt.seed = arr(sd, np.uint64, B)
        if accept_uniform is not None:
            opt.accept_uniform = arr(accept_uniform, np.float64, n_d)
        if draw_uniform is not None:
            opt.draw_uniform = arr(draw_uniform, np.float64, n_d + B)
        if stop_lists is not None:
            offs, toks = stop_lists if isinstance(stop_lists, tuple) else stop_csr(stop_lists)
            opt.stop_offsets = arr(offs, np.int32, B + 1)
            opt.stop_tokens = arr(toks, np.int32, np.size(toks)) if np.size(toks) else None
            opt.n_stop_tokens = int(np.size(toks))
        if budget is not None:
            opt.budget = arr(budget, np.int32, B)
        if draft_probs is not None:
            opt.draft_probs = arr(draft_probs, np.float32, n_d * V)
        if top_k is not None:
            opt.top_k = arr(np.broadcast_to(np.asarray(top_k, dtype=np.int32), (B,)), np.int32, B)
        if top_p_milli is not None:
            opt.top_p_milli = arr(np.broadcast_to(np.asarray(top_p_milli, dtype=np.int32), (B,)), np.int32, B)
        if top_k is not None or top_p_milli is not None:
            res["kept_tokens"] = np.full(n_d + B + n_d, -7, dtype=np.int32)
            opt.kept_tokens = _ptr(res["kept_tokens"])
        res["emitted_len"] = np.full(B, -7, dtype=np.int32)
        opt.emitted_len = _ptr(res["emitted_len"])
        rc = lib.oracle_verify_opts(_ptr(target), _ptr(draft), dt, _ptr(draft_tokens), _ptr(cu), B, n_d, V,
                                    float(temperature) if np.ndim(temperature) == 0 else 0.0,
                                    int(seed) & 0xFFFFFFFFFFFFFFFF if np.ndim(seed) == 0 else 0,
                                    ctypes.byref(opt), _ptr(acc), _ptr(out), dg_p)
    elif np.ndim(temperature) == 0 and np.ndim(seed) == 0:
        rc = lib.oracle_verify(_ptr(target), _ptr(draft), dt, _ptr(draft_tokens), _ptr(cu), B, n_d, V,
                               float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(acc), _ptr(out), dg_p)
    else:
        t_each = np.ascontiguousarray(np.broadcast_to(np.asarray(temperature, dtype=np.float64), (B,)))
        s_each = np.ascontiguousarray(np.broadcast_to(
            np.asarray([int(x) & 0xFFFFFFFFFFFFFFFF for x in np.ravel(seed)], dtype=np.uint64)
            if np.ndim(seed) else np.uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), (B,)))
        rc = lib.oracle_verify_profiled(_ptr(target), _ptr(draft), dt, _ptr(draft_tokens), _ptr(cu), B, n_d, V,
                                        _ptr(t_each), _ptr(s_each), _ptr(acc), _ptr(out), dg_p)
    if rc != 0:
        raise ValueError(f"oracle_verify rejected its arguments (status {rc})")
    return res


def philox4x32_10(counter, key) -> np.ndarray:
    lib = load()
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox_block(seed: int, request: int, position: int) -> np.ndarray:
    lib = load()
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox_block(int(seed) & 0xFFFFFFFFFFFFFFFF, request, position, _ptr(out))
    return out


def philox_grid(seed: int, n_requests: int, n_positions: int) -> np.ndarray:
    """Blocks for every (request, position) pair, shape (n_requests, n_positions, 4)."""
    out = np.zeros((n_requests, n_positions, 4), dtype=np.uint32)
    load().oracle_philox_grid(int(seed) & 0xFFFFFFFFFFFFFFFF, n_requests, n_positions, _ptr(out))
    return out


def row_lse(row: np.ndarray, temperature: float) -> float:
    row = np.ascontiguousarray(row)
    return load().oracle_row_lse(_ptr(row), _dtype_code(row), 0, row.shape[-1], float(temperature))


def row_argmax(row: np.ndarray) -> int:
    row = np.ascontiguousarray(row)
    return load().oracle_row_argmax(_ptr(row), _dtype_code(row), 0, row.shape[-1])


def truncate_row(row: np.ndarray, temperature: float, top_k: int = 0, top_p_milli: int = 1000,
                 lib_path: str = LIBRARY) -> dict:
    """The tokens one row keeps under a sampling profile: keep (V,) bool, n kept, lse_kept =
    ln sum over kept tokens of exp(z / T), and the top-p decision margin."""
    row = np.ascontiguousarray(row)
    V = row.shape[-1]
    keep = np.zeros(V, dtype=np.uint8)
    lse, margin = ctypes.c_double(), ctypes.c_double()
    n = load(lib_path).oracle_truncate_row(_ptr(row), _dtype_code(row), 0, V, float(temperature), int(top_k),
                                   int(top_p_milli), _ptr(keep), ctypes.byref(lse), ctypes.byref(margin))
    if n < 0:
        raise MemoryError("oracle_truncate_row ran out of memory")
    return {"keep": keep.astype(bool), "n": int(n), "lse_kept": lse.value, "margin": margin.value}


def num_threads() -> int:
    return load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    load().oracle_set_num_threads(n)


def verify_tree(target: np.ndarray, draft: np.ndarray | None, draft_tokens: np.ndarray, parents: np.ndarray,
                cu: np.ndarray, temperature: float, seed: int, diag: bool = False, lib_path: str = LIBRARY,
                draft_row: np.ndarray | None = None) -> dict:
    """Run the oracle's token-tree verification (oracle_verify_tree) on one batch.

    target: (n_nodes + B, V), row cu[i] + i at request i's root and cu[i] + i + n + 1 after node n;
    draft: (n_draft_rows, V), the distributions the nodes were drawn from (None when temperature == 0):
    row draft_row[cu[i] + n] for node n, or row cu[i] + n without draft_row (n_draft_rows = n_nodes);
    draft_tokens, parents: (n_nodes,) int32, parents in [-1, n - 1] within the request; cu: (B + 1,)
    node offsets.  Returns accepted_len (B,), out_tokens (n_nodes + B,),
    accepted_nodes (n_nodes,), and with ``diag`` the LSEs, argmaxes, ratios and accept margins of
    the nodes tested (NaN elsewhere), cdf margins, residual masses and terminal kinds.
    """
    lib = load(lib_path)
    target = np.ascontiguousarray(target)
    dt = _dtype_code(target)
    if draft is not None:
        draft = np.ascontiguousarray(draft)
        if _dtype_code(draft) != dt:
            raise TypeError("target and draft must share a dtype")
    draft_tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    B = cu.shape[0] - 1
    n = draft_tokens.shape[0]
    V = target.shape[1]
    if target.shape[0] != n + B or parents.shape[0] != n:
        raise ValueError("target must have n_nodes + B rows and parents n_nodes entries")
    if draft_row is not None:
        draft_row = np.ascontiguousarray(draft_row, dtype=np.int32)
        if draft_row.shape[0] != n:
            raise ValueError("draft_row must have n_nodes entries")
    n_dr = n if draft_row is None else (draft.shape[0] if draft is not None else int(draft_row.max(initial=-1)) + 1)
    acc = np.full(B, -7, dtype=np.int32)
    out = np.full(n + B, -7, dtype=np.int32)
    nodes = np.full(n, -7, dtype=np.int32)
    res: dict = {"accepted_len": acc, "out_tokens": out, "accepted_nodes": nodes}
    dg_p = None
    if diag:
        res.update(
            target_lse=np.full(n + B, np.nan), draft_lse=np.full(n, np.nan),
            target_argmax=np.full(n + B, -1, dtype=np.int32), ratio=np.full(n, np.nan),
            accept_margin=np.full(n, np.nan), cdf_margin=np.full(B, np.nan),
            resid_mass=np.full(B, np.nan), terminal_kind=np.full(B, -9, dtype=np.int32),
            filter_margin=np.full(2 * n + B, np.inf),
        )
        dg = _Diag(*[_ptr(res[f]) for f, _ in _Diag._fields_])
        dg_p = ctypes.pointer(dg)
    rc = lib.oracle_verify_tree(_ptr(target), _ptr(draft), dt, _ptr(draft_tokens), _ptr(parents), _ptr(draft_row), n_dr,
                                _ptr(cu), B, n, V,
                                float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(acc), _ptr(out), _ptr(nodes),
                                dg_p)
    if rc != 0:
        raise ValueError(f"oracle_verify_tree rejected the batch ({rc})")
    return res
