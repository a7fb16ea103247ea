"""SDCP's verifier uniforms from Python's standard hmac and hashlib modules.

TEST INFRASTRUCTURE ONLY: the independent side against which the library's host implementation is
checked.  "Speculative Decoding Coordination Protocol (SDCP)", section "Acceptance Rules", Rule 2:
each value is the first 53 bits of HMAC-SHA-256 keyed with the profile's seed (eight octets,
network byte order) over "SDCP-VERIFY-1" || 0x00 || session || uint32(round) || uint32(i) ||
uint8(purpose), divided by 2^53; purpose 0 is the acceptance test, 1 the draw of the extra token.
Readings: the uint32 fields are in network byte order like the seed, and positions i count from 1
as SDCP numbers p[1..M+1]; the extra token is drawn at its own position (the first rejected one,
or M + 1).
"""
from __future__ import annotations

import hashlib
import hmac

import numpy as np


def uniform(seed: int, session: bytes, round_: int, position: int, purpose: int) -> float:
    key = int(seed).to_bytes(8, "big")
    msg = (b"SDCP-VERIFY-1" + b"\x00" + bytes(session) + int(round_).to_bytes(4, "big")
           + int(position).to_bytes(4, "big") + bytes([purpose]))
    mac = hmac.new(key, msg, hashlib.sha256).digest()
    return (int.from_bytes(mac[:8], "big") >> 11) / 2.0**53


def batch_uniforms(cu, seeds, sessions, rounds) -> tuple[np.ndarray, np.ndarray]:
    """accept_uniform [cu[B]] (position j + 1, purpose 0) and draw_uniform [cu[B] + B] (position
    t + 1, purpose 1) in the layout the verifier takes."""
    cu = np.asarray(cu)
    B = cu.shape[0] - 1
    r = np.zeros(int(cu[-1]))
    u = np.zeros(int(cu[-1]) + B)
    for i in range(B):
        K = int(cu[i + 1] - cu[i])
        sess = bytes(np.asarray(sessions[i], dtype=np.uint8))
        for j in range(K):
            r[cu[i] + j] = uniform(int(seeds[i]), sess, int(rounds[i]), j + 1, 0)
        for t in range(K + 1):
            u[cu[i] + i + t] = uniform(int(seeds[i]), sess, int(rounds[i]), t + 1, 1)
    return r, u
