// Post-verification commit of a ragged batch ("M7.8 - Speculative Serving", sections 0x03C and
// 0x03D: unpad, append, repad; section 0x09 for the lengths after a round).  sdv_commit is one
// workgroup: a block-wide exclusive scan of the emitted counts, then every request copies its
// emitted tokens to their packed place and writes its new lengths.  The work is a few loads per
// request; what it costs is latency, so one workgroup with the scan in shared memory is the whole
// design.  sdv_repad writes the rectangular form, one thread per cell.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sdv.h"

namespace commit_impl {

constexpr int kThreads = 1024;
constexpr int kWave = 64;

// Emitted tokens of request i: emitted_len[i] if given, else a_i + 1; 0 for a rejected request or
// one whose offsets fall outside [0, n_d] (its slots could not be named).
__device__ __forceinline__ int32_t emitted_of(const int32_t* cu, const int32_t* acc, const int32_t* emitted, int32_t i,
                                              int64_t n_d) {
  const int32_t a = acc[i], lo = cu[i], hi = cu[i + 1], K = hi - lo;
  if (a < 0 || lo < 0 || hi > n_d || K < 0 || K > SDV_MAX_DEPTH || a > K) return 0;
  const int32_t n = emitted ? emitted[i] : a + 1;
  return n < 0 ? 0 : (n > a + 1 ? a + 1 : n);
}

// Writes land only below capacity = n_d + B, the size of new_tokens / new_positions: offsets that
// are not non-decreasing could otherwise make the emitted total exceed it.
__global__ __launch_bounds__(kThreads) void commit_kernel(int32_t B, int64_t n_d, const int32_t* __restrict__ cu,
                                                          const int32_t* __restrict__ acc,
                                                          const int32_t* __restrict__ emitted,
                                                          const int32_t* __restrict__ out_tokens,
                                                          const int32_t* __restrict__ prefix, int32_t* new_offsets,
                                                          int32_t* new_tokens, int32_t* new_positions, int32_t* lengths,
                                                          int32_t* next_token, int32_t* next_position) {
  __shared__ int32_t wave_sums[kThreads / kWave];
  __shared__ int32_t carry_s;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int32_t s = 0; s < B; s += kThreads) {  // tiles of 1024 requests, every thread in every pass
    const int32_t i = s + t;
    const int32_t n = i < B ? emitted_of(cu, acc, emitted, i, n_d) : 0;
    // exclusive scan: within the wave, then over the wave totals
    int32_t incl = n;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int32_t up = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += up;
    }
    if (lane == kWave - 1) wave_sums[wave] = incl;
    __syncthreads();
    int32_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wave_sums[w];
    const int32_t off = before + incl - n;
    if (i < B) {
      new_offsets[i] = off;
      const int32_t a = acc[i], K = cu[i + 1] - cu[i], P = prefix[i];
      const int32_t base = cu[i] + i;
      for (int32_t j = 0; j < n; ++j) {
        if ((int64_t)off + j >= n_d + B) break;
        new_tokens[off + j] = out_tokens[base + j];
        new_positions[off + j] = P + j;
      }
      const int32_t E = max(min(n, a), 0), F = (n > 0 && n == a + 1) ? 1 : 0;  // a rejected request: E = F = 0
      const int32_t km1 = K > 0 ? K - 1 : 0;
      lengths[3 * i] = P + E + F;
      lengths[3 * i + 1] = P + E;
      lengths[3 * i + 2] = P + (E < km1 ? E : km1);
      next_token[i] = n > 0 ? out_tokens[base + n - 1] : -1;
      next_position[i] = n > 0 ? P + n - 1 : -1;
    }
    __syncthreads();
    if (t == kThreads - 1) carry_s = off + n;  // the last thread's inclusive prefix is the tile total
    __syncthreads();
  }
  if (t == 0) new_offsets[B] = carry_s;
}

// Repad (section 0x03D): row i of the [B, width] batch holds request i's prefix followed by its
// emitted tokens at logical positions 0 .. L_i - 1, padding elsewhere (pad_id, position -1, mask 0).
// One thread per cell, grid-stride over B * width; each thread recomputes its row's few scalars
// (cached loads), so no cell waits for another and the writes stay coalesced along the row.
constexpr int kRepadThreads = 256;

__global__ __launch_bounds__(kRepadThreads) void repad_kernel(int32_t B, int64_t n_d, const int32_t* __restrict__ cu,
                                                              const int32_t* __restrict__ acc,
                                                              const int32_t* __restrict__ emitted,
                                                              const int32_t* __restrict__ out_tokens,
                                                              const int32_t* __restrict__ po,
                                                              const int32_t* __restrict__ ptok, int64_t n_prefix,
                                                              int32_t width, int32_t pad_id, int32_t left_pad,
                                                              int32_t* token_ids, int32_t* position_ids, uint8_t* mask,
                                                              int32_t* row_len) {
  const int64_t cells = (int64_t)B * width;
  for (int64_t e = (int64_t)blockIdx.x * kRepadThreads + threadIdx.x; e < cells;
       e += (int64_t)gridDim.x * kRepadThreads) {
    const int32_t i = (int32_t)(e / width), c = (int32_t)(e - (int64_t)i * width);
    const int32_t lo = po[i], hi = po[i + 1];
    const bool ok = lo >= 0 && hi >= lo && (int64_t)hi <= n_prefix;
    const int32_t P = ok ? hi - lo : 0;
    const int32_t n = ok ? emitted_of(cu, acc, emitted, i, n_d) : 0;
    const int64_t L = (int64_t)P + n;
    if (c == 0) row_len[i] = ok ? (int32_t)L : -1;
    int32_t tok = pad_id, pos = -1;
    uint8_t m = 0;
    if (ok && L <= width) {
      const int64_t k = c - (left_pad ? width - L : 0);  // the cell's logical position
      if (k >= 0 && k < L) {
        tok = k < P ? ptok[lo + k] : out_tokens[(int64_t)cu[i] + i + (k - P)];
        pos = (int32_t)k;
        m = 1;
      }
    }
    token_ids[e] = tok;
    position_ids[e] = pos;
    mask[e] = m;
  }
}

}  // namespace commit_impl

extern "C" int sdv_commit(int32_t B, int64_t n_draft_rows, const int32_t* ragged_offsets, const int32_t* accepted_len,
                          const int32_t* emitted_len, const int32_t* out_tokens, const int32_t* prefix_len,
                          int32_t* new_offsets, int32_t* new_tokens, int32_t* new_positions, int32_t* lengths,
                          int32_t* next_token, int32_t* next_position, void* stream) {
  if (B < 1 || n_draft_rows < 0 || !ragged_offsets || !accepted_len || !out_tokens || !prefix_len || !new_offsets ||
      !new_tokens || !new_positions || !lengths || !next_token || !next_position)
    return SDV_ERR_INVALID_ARG;
  if (n_draft_rows + B > INT32_MAX) return SDV_ERR_LIMIT;
  hipLaunchKernelGGL(commit_impl::commit_kernel, dim3(1), dim3(commit_impl::kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), B, n_draft_rows, ragged_offsets, accepted_len,
                     emitted_len, out_tokens,
                     prefix_len, new_offsets, new_tokens, new_positions, lengths, next_token, next_position);
  return hipGetLastError() == hipSuccess ? SDV_OK : SDV_ERR_HIP;
}

extern "C" int sdv_repad(int32_t B, int64_t n_draft_rows, const int32_t* ragged_offsets, const int32_t* accepted_len,
                         const int32_t* emitted_len, const int32_t* out_tokens, const int32_t* prefix_offsets,
                         const int32_t* prefix_tokens, int64_t n_prefix_tokens, int32_t width, int32_t pad_id,
                         int32_t left_pad, int32_t* token_ids, int32_t* position_ids, uint8_t* mask, int32_t* row_len,
                         void* stream) {
  if (B < 1 || n_draft_rows < 0 || n_prefix_tokens < 0 || width < 1 || !ragged_offsets || !accepted_len ||
      !out_tokens || !prefix_offsets || (n_prefix_tokens > 0 && !prefix_tokens) || !token_ids || !position_ids ||
      !mask || !row_len)
    return SDV_ERR_INVALID_ARG;
  if (n_draft_rows + B > INT32_MAX || n_prefix_tokens > INT32_MAX - 128 || (int64_t)B * width > ((int64_t)1 << 40))
    return SDV_ERR_LIMIT;
  const int64_t cells = (int64_t)B * width;
  const int64_t blocks = (cells + commit_impl::kRepadThreads - 1) / commit_impl::kRepadThreads;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(commit_impl::repad_kernel, dim3(grid), dim3(commit_impl::kRepadThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), B, n_draft_rows, ragged_offsets, accepted_len, emitted_len,
                     out_tokens, prefix_offsets, prefix_tokens, n_prefix_tokens, width, pad_id, left_pad != 0,
                     token_ids, position_ids, mask, row_len);
  return hipGetLastError() == hipSuccess ? SDV_OK : SDV_ERR_HIP;
}
