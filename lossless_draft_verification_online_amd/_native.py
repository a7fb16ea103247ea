"""ctypes declarations of libsdv.so (include/sdv.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

from .build import LIBRARY

SDV_BF16, SDV_FP32 = 0, 1
SDV_MAX_DEPTH = 64
SDV_MAX_EVENTS = 4
SDV_NOALLOC_SCRATCH_BYTES = 8 << 20
STATUS = {0: "SDV_OK", -1: "SDV_ERR_INVALID_ARG", -2: "SDV_ERR_UNSUPPORTED", -3: "SDV_ERR_LIMIT",
          -4: "SDV_ERR_WORKSPACE", -5: "SDV_ERR_HIP"}
TERM_GREEDY, TERM_BONUS, TERM_RESIDUAL, TERM_RESIDUAL_EMPTY, TERM_NONE, TERM_BAD = 0, 1, 2, 3, 4, -1


class SdvDiag(ctypes.Structure):
    _fields_ = [
        ("target_lse", ctypes.c_void_p),
        ("draft_lse", ctypes.c_void_p),
        ("target_argmax", ctypes.c_void_p),
        ("ratio", ctypes.c_void_p),
        ("accept_uniform", ctypes.c_void_p),
        ("draw_uniform", ctypes.c_void_p),
        ("terminal_kind", ctypes.c_void_p),
        ("events", ctypes.c_void_p * SDV_MAX_EVENTS),
        ("target_logit", ctypes.c_void_p),
        ("draft_logit", ctypes.c_void_p),
        ("terminal_mass", ctypes.c_void_p),
    ]


class SdvError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


class SdvOptions(ctypes.Structure):
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
        ("verdict_split", ctypes.c_int32),
    ]


_LIB = None

_VERIFY_ARGS = [
    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,  # target, draft, tokens, offsets
    ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,      # B, n_draft_rows, V, dtype
    ctypes.c_double, ctypes.c_uint64,                                     # temperature, seed
    ctypes.c_void_p, ctypes.c_void_p,                                     # accepted_len, out_tokens
    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,                    # workspace, bytes, stream
]


def lib(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libsdv.so.  There is no fallback: a missing library is an error."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
    L = ctypes.CDLL(path)
    L.sdv_workspace_bytes.restype = ctypes.c_size_t
    L.sdv_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    L.sdv_verify.restype = ctypes.c_int
    L.sdv_verify.argtypes = list(_VERIFY_ARGS)
    L.sdv_verify_noalloc.restype = ctypes.c_int
    L.sdv_verify_noalloc.argtypes = list(_VERIFY_ARGS[:12]) + [ctypes.c_void_p]
    L.sdv_noalloc_bytes.restype = ctypes.c_size_t
    L.sdv_noalloc_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    L.sdv_verify_ex.restype = ctypes.c_int
    L.sdv_verify_ex.argtypes = list(_VERIFY_ARGS) + [ctypes.POINTER(SdvDiag)]
    L.sdv_verify_tree.restype = ctypes.c_int
    L.sdv_verify_tree.argtypes = ([ctypes.c_void_p] * 6 + [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_double, ctypes.c_uint64] + [ctypes.c_void_p] * 4 +
                                  [ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(SdvDiag)])
    L.sdv_verify_profiled.restype = ctypes.c_int
    L.sdv_verify_profiled.argtypes = (list(_VERIFY_ARGS[:8]) + [ctypes.c_void_p, ctypes.c_void_p]
                                      + list(_VERIFY_ARGS[10:]) + [ctypes.POINTER(SdvDiag)])
    L.sdv_verify_opts.restype = ctypes.c_int
    L.sdv_verify_opts.argtypes = (list(_VERIFY_ARGS[:10]) + [ctypes.POINTER(SdvOptions)] + list(_VERIFY_ARGS[10:])
                                  + [ctypes.POINTER(SdvDiag)])
    L.sdv_sdcp_uniforms.restype = ctypes.c_int
    L.sdv_sdcp_uniforms.argtypes = [ctypes.c_int32] + [ctypes.c_void_p] * 6
    L.sdv_commit.restype = ctypes.c_int
    L.sdv_commit.argtypes = [ctypes.c_int32, ctypes.c_int64] + [ctypes.c_void_p] * 12
    L.sdv_repad.restype = ctypes.c_int
    L.sdv_repad.argtypes = ([ctypes.c_int32, ctypes.c_int64] + [ctypes.c_void_p] * 6 +
                            [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 5)
    L.sdv_philox4x32_10.restype = ctypes.c_int
    L.sdv_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.sdv_philox_uniforms.restype = ctypes.c_int
    L.sdv_philox_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.sdv_status_string.restype = ctypes.c_char_p
    L.sdv_read_yardstick.restype = ctypes.c_int
    L.sdv_read_yardstick.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.sdv_read_ceiling.restype = ctypes.c_int
    L.sdv_read_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.sdv_status_string.argtypes = [ctypes.c_int]
    L.sdv_abi_version.restype = ctypes.c_int
    L.sdv_abi_version.argtypes = []
    _LIB = L
    return L
