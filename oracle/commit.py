"""Post-verification commit of a ragged batch, written plainly (loops over requests).

TEST INFRASTRUCTURE ONLY: the reference the library's commit kernel is checked against.

"M7.8 - Speculative Serving", sections 0x03C and 0x03D: after verification every request grows by
a ragged number of tokens; the batch is unpadded, each request's emitted tokens are appended to its
logical sequence at contiguous positions (the position invariant: positions P_i, P_i + 1, ... with
no gap), and the batch is repadded.  Section 0x09 ("EOS and length-limit stopping") gives the
lengths after a round: with E_i the accepted drafts actually emitted and F_i = 1 when the extra
token (correction or bonus) is emitted,
    L_out = P + E + F,   L_target = P + E,   L_draft = P + min(E, K - 1).
Reading: for a request with no drafts (K = 0) the draft length does not change, L_draft = P.
"""
from __future__ import annotations

import numpy as np


def commit(cu, accepted_len, out_tokens, prefix_len, emitted_len=None) -> dict:
    cu = np.asarray(cu, dtype=np.int64)
    acc = np.asarray(accepted_len, dtype=np.int64)
    out = np.asarray(out_tokens)
    P = np.asarray(prefix_len, dtype=np.int64)
    B = cu.shape[0] - 1
    n_emit = np.zeros(B, dtype=np.int64)
    E = np.zeros(B, dtype=np.int64)
    F = np.zeros(B, dtype=np.int64)
    for i in range(B):
        K = int(cu[i + 1] - cu[i])
        a = int(acc[i])
        if a < 0 or K < 0 or K > 64:
            continue  # a rejected request emits nothing
        n = a + 1 if emitted_len is None else int(emitted_len[i])
        n = min(max(n, 0), a + 1)
        n_emit[i] = n
        E[i] = min(n, a)
        F[i] = int(n == a + 1)
    offsets = np.concatenate([[0], np.cumsum(n_emit)]).astype(np.int32)
    tokens = np.full(int(offsets[-1]), -1, dtype=np.int32)
    positions = np.full(int(offsets[-1]), -1, dtype=np.int32)
    next_token = np.full(B, -1, dtype=np.int32)
    next_position = np.full(B, -1, dtype=np.int32)
    lengths = np.zeros((B, 3), dtype=np.int32)
    for i in range(B):
        K = int(cu[i + 1] - cu[i])
        base = int(cu[i]) + i
        for j in range(int(n_emit[i])):
            tokens[offsets[i] + j] = out[base + j]
            positions[offsets[i] + j] = P[i] + j
        lengths[i] = (P[i] + E[i] + F[i], P[i] + E[i], P[i] + min(E[i], max(K - 1, 0)))
        if n_emit[i] > 0:
            next_token[i] = tokens[offsets[i + 1] - 1]
            next_position[i] = positions[offsets[i + 1] - 1]
    return {"offsets": offsets, "tokens": tokens, "positions": positions, "lengths": lengths,
            "next_token": next_token, "next_position": next_position}


def repad(cu, accepted_len, out_tokens, prefix_offsets, prefix_tokens, width, pad_id, left_pad,
          emitted_len=None) -> dict:
    """The repad step of section 0x03D: request i's logical sequence is its prefix (prefix_tokens
    [prefix_offsets[i] : prefix_offsets[i + 1]]) followed by the tokens it emitted this round (as
    ``commit`` finds them), and row i of a [B, width] batch holds that sequence at logical positions
    0 .. L_i - 1 with padding in the other columns: token pad_id, position -1 (padding takes no
    logical position, section 0x03C's position invariant) and mask 0.  With left_pad the padding
    comes first, so every row ends in the last column.  A row whose sequence is longer than width
    is all padding and reports its length L_i > width; a row whose prefix offsets are decreasing or
    outside [0, len(prefix_tokens)] is all padding and reports -1."""
    po = np.asarray(prefix_offsets, dtype=np.int64)
    pt = np.asarray(prefix_tokens, dtype=np.int64).reshape(-1)
    B = po.shape[0] - 1
    new = commit(cu, accepted_len, out_tokens, np.zeros(B, dtype=np.int64), emitted_len)
    token_ids = np.full((B, width), pad_id, dtype=np.int32)
    position_ids = np.full((B, width), -1, dtype=np.int32)
    mask = np.zeros((B, width), dtype=np.uint8)
    row_len = np.zeros(B, dtype=np.int32)
    for i in range(B):
        lo, hi = int(po[i]), int(po[i + 1])
        if lo < 0 or hi < lo or hi > pt.shape[0]:
            row_len[i] = -1
            continue
        logical = list(pt[lo:hi]) + list(new["tokens"][new["offsets"][i]:new["offsets"][i + 1]])
        L = len(logical)
        row_len[i] = L
        if L > width:
            continue
        first = width - L if left_pad else 0
        for k in range(L):
            token_ids[i, first + k] = logical[k]
            position_ids[i, first + k] = k
            mask[i, first + k] = 1
    return {"token_ids": token_ids, "position_ids": position_ids, "mask": mask, "row_len": row_len}
