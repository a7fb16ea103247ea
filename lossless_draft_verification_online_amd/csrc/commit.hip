// Post-verification commit of a ragged batch ("M7.8 - Speculative Serving", sections 0x03C and
// 0x03D: unpad, append, repad; section 0x09 for the lengths after a round).  One workgroup: a
// block-wide exclusive scan of the emitted counts, then every request copies its emitted tokens to
// their packed place and writes its new lengths.  The work is a few loads per request; what it
// costs is latency, so one workgroup with the scan in shared memory is the whole design.
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
