// Batched speculative-sampling verification on MI355X (gfx950): kernels and the C ABI.
//
// The step verifies every request of a ragged batch at once (SDCP "Verification and Commit",
// steps 5 to 7; Rule 1 and Rule 2 of its section "Acceptance Rules"; the r <= p/q test of
// "SOTA-227", section "What to do").  It runs as three kernels on the caller's stream:
//
//   1. row pass      one wave64 per 16 KiB chunk of every logit row: a single coalesced read of
//                    the chunk; at T > 0 it records the chunk's max-based exponent reference and
//                    its sum of 2^(z k - ref) (k = log2(e)/T), at T = 0 the chunk's max and the
//                    smallest index reaching it.  This kernel carries essentially all HBM traffic.
//   2. accept scan   one wave64 per request: lane j folds the chunk records of its target and
//                    draft rows into log-normalisers (fp64), gathers the two logits at the draft
//                    token, forms p/q, draws r from Philox (seed; j, request) and the wave ballot
//                    yields the first rejection.  Greedy requests finish here.
//   3. terminal draw one workgroup per request (T > 0 only): chunk masses of the residual
//                    max(p - q, 0) of the rejected position (re-reading that row pair), or of p
//                    at the bonus position (from the row pass records, no re-read); the chunk
//                    holding u * S is found by prefix sum and searched element by element.
//
// No matrix cores are involved: nothing here is a contraction.  The roofline is HBM bandwidth.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <climits>

#include "../../include/sdv.h"
#include "sdv_device.hpp"

namespace sdv {

// Per-request hand-off from the accept scan to the terminal draw.
struct ReqInfo {
  int32_t kind;  // sdv_terminal_kind
  int32_t t;     // drawn position
  int32_t trow;  // target row of the drawn position
  int32_t drow;  // draft row of the drawn position (residual draws), else -1
  float u;       // draw uniform
  float ref_t;   // weights are 2^(z_t k - ref_t): ref_t is the largest chunk reference of the target row
  float e_hi;    // draft side: q-weights are 2^(z_d k - e), e = ref_t + log2-normaliser(draft) - (target),
  float e_lo;    //   carried as e_hi + e_lo to keep fp64 accuracy
};

struct DiagPtrs {
  double* target_lse;
  double* draft_lse;
  int32_t* target_argmax;
  double* ratio;
  float* accept_uniform;
  float* draw_uniform;
  int32_t* terminal_kind;
};

constexpr double kLn2 = 0.69314718055994530942;

// ============================================================================ 1. row pass

template <class E, bool kGreedy>
__device__ inline void finish_chunk_greedy(float best, int32_t idx, float2* out, int lane) {
  wave_argmax(best, idx);
  if (lane == 0) *out = make_float2(best, __int_as_float(idx));
}

// 16-byte vector path: every row starts 16-byte aligned (row bytes and base pointers are multiples of 16).
template <class E, bool kGreedy>
__global__ __launch_bounds__(256) void row_pass_vec(const void* __restrict__ target, const void* __restrict__ draft,
                                                    int32_t n_target_rows, int32_t V, int32_t n_chunks,
                                                    int64_t n_units, float k2, float2* __restrict__ part) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t unit = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (unit >= n_units) return;
  const int32_t row = (int32_t)(unit / n_chunks);
  const int32_t chunk = (int32_t)(unit - (int64_t)row * n_chunks);
  const char* rp = row < n_target_rows ? row_ptr<E>(target, row, V) : row_ptr<E>(draft, row - n_target_rows, V);
  const int32_t c0 = chunk * E::kChunk;
  const int32_t nvec = min(E::kChunk, V - c0) / E::kPerVec;
  const u32x4* vp = reinterpret_cast<const u32x4*>(rp + (int64_t)c0 * E::kBytes);

  u32x4 buf[kVecPerLane];
#pragma unroll
  for (int k = 0; k < kVecPerLane; ++k) {
    const int vi = lane + kWave * k;
    buf[k] = vi < nvec ? vp[vi] : u32x4{E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord};
  }

  if constexpr (kGreedy) {
    float best = -INFINITY;
    int32_t idx = INT32_MAX;
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) {
      float f[E::kPerVec];
      E::unpack(buf[k], f);
      const int32_t e0 = c0 + (lane + kWave * k) * E::kPerVec;
#pragma unroll
      for (int e = 0; e < E::kPerVec; ++e) {
        if (f[e] > best) {  // ascending within the lane: the first maximum is kept
          best = f[e];
          idx = e0 + e;
        }
      }
    }
    finish_chunk_greedy<E, kGreedy>(best, idx, part + unit, lane);
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) {
      float f[E::kPerVec];
      E::unpack(buf[k], f);
#pragma unroll
      for (int e = 0; e < E::kPerVec; ++e) m = fmaxf(m, f[e]);
    }
    m = wave_max(m);
    float ref = -INFINITY, s = 0.0f;
    if (m != -INFINITY) {
      ref = m * k2;
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < kVecPerLane; ++k) {
        float f[E::kPerVec];
        E::unpack(buf[k], f);
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e) f[e] = fast_exp2(fmaf(f[e], k2, -ref));
        acc[k & 3] += tree_sum(f);
      }
      s = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
    }
    if (lane == 0) part[unit] = make_float2(ref, s);
  }
}

// Element-wise path for rows that are not 16-byte aligned: two passes over the chunk.
template <class E, bool kGreedy>
__global__ __launch_bounds__(256) void row_pass_scalar(const void* __restrict__ target,
                                                       const void* __restrict__ draft, int32_t n_target_rows,
                                                       int32_t V, int32_t n_chunks, int64_t n_units, float k2,
                                                       float2* __restrict__ part) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t unit = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (unit >= n_units) return;
  const int32_t row = (int32_t)(unit / n_chunks);
  const int32_t chunk = (int32_t)(unit - (int64_t)row * n_chunks);
  const char* rp = row < n_target_rows ? row_ptr<E>(target, row, V) : row_ptr<E>(draft, row - n_target_rows, V);
  const int32_t c0 = chunk * E::kChunk;
  const int32_t c1 = min(c0 + E::kChunk, V);
  if constexpr (kGreedy) {
    float best = -INFINITY;
    int32_t idx = INT32_MAX;
    for (int32_t v = c0 + lane; v < c1; v += kWave) {
      const float z = E::at(rp, v);
      if (z > best) {
        best = z;
        idx = v;
      }
    }
    finish_chunk_greedy<E, kGreedy>(best, idx, part + unit, lane);
  } else {
    float m = -INFINITY;
    for (int32_t v = c0 + lane; v < c1; v += kWave) m = fmaxf(m, E::at(rp, v));
    m = wave_max(m);
    float ref = -INFINITY, s = 0.0f;
    if (m != -INFINITY) {
      ref = m * k2;
      for (int32_t v = c0 + lane; v < c1; v += kWave) s += fast_exp2(fmaf(E::at(rp, v), k2, -ref));
      s = wave_sum(s);
    }
    if (lane == 0) part[unit] = make_float2(ref, s);
  }
}

// ============================================================================ 2. accept scan

struct Frame {
  double l2;  // log2 sum_v 2^(z_v k)
  float ref;  // largest chunk reference of the row
};

// Fold the chunk records of one row: l2 = R + log2(sum_c s_c 2^(ref_c - R)), R = max_c ref_c.
__device__ inline Frame fold_row(const float2* __restrict__ p, int32_t n_chunks) {
  float R = -INFINITY;
  for (int32_t c = 0; c < n_chunks; ++c) R = fmaxf(R, p[c].x);
  if (R == -INFINITY) return {-(double)INFINITY, R};
  double s = 0.0;
  for (int32_t c = 0; c < n_chunks; ++c) s += (double)p[c].y * exp2((double)p[c].x - (double)R);
  return {(double)R + log2(s), R};
}

// Chunk maxima in ascending order with a strict comparison: the smallest index of the row maximum.
__device__ inline int32_t fold_argmax(const float2* __restrict__ p, int32_t n_chunks) {
  float best = p[0].x;
  int32_t idx = __float_as_int(p[0].y);
  for (int32_t c = 1; c < n_chunks; ++c) {
    if (p[c].x > best) {
      best = p[c].x;
      idx = __float_as_int(p[c].y);
    }
  }
  return idx == INT32_MAX ? 0 : idx;  // a row of -inf only: index 0
}

__device__ inline void reject_request(int32_t i, int32_t trow0, int K, int lane, int32_t* accepted_len,
                                      int32_t* out_tokens, ReqInfo* info, const DiagPtrs& dg) {
  for (int j = lane; j <= K; j += kWave) out_tokens[trow0 + j] = -1;
  if (lane == 0) {
    accepted_len[i] = -1;
    info[i].kind = SDV_TERM_BAD;
    if (dg.terminal_kind) dg.terminal_kind[i] = SDV_TERM_BAD;
  }
}

template <class E, bool kGreedy>
__global__ __launch_bounds__(64) void accept_scan(const void* __restrict__ target, const void* __restrict__ draft,
                                                  const int32_t* __restrict__ tokens, const int32_t* __restrict__ cu,
                                                  int32_t B, int32_t n_draft_rows, int32_t V, int32_t n_chunks,
                                                  float k2, uint64_t seed, const float2* __restrict__ part,
                                                  int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
                                                  ReqInfo* __restrict__ info, DiagPtrs dg) {
  const int32_t i = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t lo = cu[i], hi = cu[i + 1];
  const int64_t K64 = (int64_t)hi - (int64_t)lo;
  if (lo < 0 || hi > n_draft_rows || K64 < 0 || K64 > SDV_MAX_DEPTH) {
    // offsets that name no valid slot range: report the request and write no slot
    if (lane == 0) {
      accepted_len[i] = -1;
      info[i].kind = SDV_TERM_BAD;
      if (dg.terminal_kind) dg.terminal_kind[i] = SDV_TERM_BAD;
    }
    return;
  }
  const int K = (int)K64;
  const int32_t n_target_rows = n_draft_rows + B;
  const int32_t trow0 = lo + i, drow0 = lo;
  const bool active = lane < K;
  const int32_t x = active ? tokens[drow0 + lane] : 0;
  if (__ballot(active && (x < 0 || x >= V)) != 0) {
    reject_request(i, trow0, K, lane, accepted_len, out_tokens, info, dg);
    return;
  }

  if constexpr (kGreedy) {
    const int32_t g = lane <= K ? fold_argmax(part + (int64_t)(trow0 + lane) * n_chunks, n_chunks) : 0;
    const uint64_t miss = __ballot(active && x != g);
    const int a = miss ? __ffsll((unsigned long long)miss) - 1 : K;
    int32_t g_a = __shfl(g, a & (kWave - 1), kWave);
    int32_t g_last = 0;
    if (K == kWave) {  // target row 64 has no lane of its own
      g_last = fold_argmax(part + (int64_t)(trow0 + kWave) * n_chunks, n_chunks);
      if (a == kWave) g_a = g_last;
    }
    for (int j = lane; j <= K; j += kWave) out_tokens[trow0 + j] = j < a ? x : (j == a ? g_a : -1);
    if (dg.target_argmax) {
      if (lane <= K) dg.target_argmax[trow0 + lane] = g;
      if (K == kWave && lane == 0) dg.target_argmax[trow0 + kWave] = g_last;
    }
    if (lane == 0) {
      accepted_len[i] = a;
      info[i].kind = SDV_TERM_GREEDY;
      if (dg.terminal_kind) dg.terminal_kind[i] = SDV_TERM_GREEDY;
    }
  } else {
    // target rows j <= K (the row at j = 64 is folded separately), draft rows j < K
    Frame ft{0.0, 0.0f}, fd{0.0, 0.0f};
    if (lane <= K) ft = fold_row(part + (int64_t)(trow0 + lane) * n_chunks, n_chunks);
    double ratio = 0.0;
    float r = 1.0f;
    bool qzero = false;
    Philox4 blk{0u, 0u, 0u, 0u};
    if (active) {
      fd = fold_row(part + (int64_t)(n_target_rows + drow0 + lane) * n_chunks, n_chunks);
      const float zt = E::at(row_ptr<E>(target, trow0 + lane, V), x);
      const float zd = E::at(row_ptr<E>(draft, drow0 + lane, V), x);
      qzero = zd == -INFINITY;
      // log2 p(x)/q(x) = (z_t - z_d) k - (l2_t - l2_d)
      const double lr2 = ((double)zt - (double)zd) * (double)k2 - (ft.l2 - fd.l2);
      ratio = exp2(lr2);
      blk = verifier_block(seed, (uint32_t)i, (uint32_t)lane);
      r = accept_uniform(blk);
    }
    if (__ballot(qzero) != 0) {  // q(x) = 0 somewhere: rejected before any uniform is used
      reject_request(i, trow0, K, lane, accepted_len, out_tokens, info, dg);
      return;
    }
    const uint64_t rej = __ballot(active && !((double)r <= ratio));
    const int a = rej ? __ffsll((unsigned long long)rej) - 1 : K;

    Frame f_last{0.0, 0.0f};
    if (K == kWave) f_last = fold_row(part + (int64_t)(trow0 + kWave) * n_chunks, n_chunks);
    const float ref_bonus = K == kWave ? f_last.ref : __shfl(ft.ref, K & (kWave - 1), kWave);
    if (a < K) {
      if (lane == a) {
        ReqInfo in;
        in.kind = SDV_TERM_RESIDUAL;
        in.t = a;
        in.trow = trow0 + a;
        in.drow = drow0 + a;
        in.u = draw_uniform(blk);
        in.ref_t = ft.ref;
        const double e = (double)ft.ref + fd.l2 - ft.l2;
        in.e_hi = (float)e;
        in.e_lo = (float)(e - (double)in.e_hi);
        info[i] = in;
      }
    } else if (lane == 0) {
      ReqInfo in;
      in.kind = SDV_TERM_BONUS;
      in.t = K;
      in.trow = trow0 + K;
      in.drow = -1;
      in.u = draw_uniform(verifier_block(seed, (uint32_t)i, (uint32_t)K));
      in.ref_t = ref_bonus;
      in.e_hi = 0.0f;
      in.e_lo = 0.0f;
      info[i] = in;
    }
    for (int j = lane; j <= K; j += kWave) out_tokens[trow0 + j] = j < a ? x : -1;
    if (lane == 0) accepted_len[i] = a;

    if (dg.target_lse && lane <= K) dg.target_lse[trow0 + lane] = ft.l2 * kLn2;
    if (dg.target_lse && K == kWave && lane == 0) dg.target_lse[trow0 + kWave] = f_last.l2 * kLn2;
    if (active) {
      if (dg.draft_lse) dg.draft_lse[drow0 + lane] = fd.l2 * kLn2;
      if (dg.ratio) dg.ratio[drow0 + lane] = ratio;
      if (dg.accept_uniform) dg.accept_uniform[drow0 + lane] = r;
    }
    if (lane == 0) {
      if (dg.terminal_kind) dg.terminal_kind[i] = a < K ? SDV_TERM_RESIDUAL : SDV_TERM_BONUS;
    }
    if (dg.draw_uniform) {
      if (a < K && lane == a) dg.draw_uniform[i] = draw_uniform(blk);
      if (a == K && lane == 0) dg.draw_uniform[i] = draw_uniform(verifier_block(seed, (uint32_t)i, (uint32_t)K));
    }
  }
}

// ============================================================================ 3. terminal draw

// Residual weight max(p - q, 0), both sides scaled by the same factor 2^(l2_t - ref_t).
__device__ inline float resid_weight(float zt, float zd, float k2, float ref_t, float e_hi, float e_lo) {
  const float p = fast_exp2(fmaf(zt, k2, -ref_t));
  const float q = fast_exp2(fmaf(zd, k2, -e_hi) - e_lo);
  return fmaxf(p - q, 0.0f);
}

__device__ inline float target_weight(float zt, float k2, float ref_t) { return fast_exp2(fmaf(zt, k2, -ref_t)); }

// Residual mass of one chunk, coalesced 16-byte loads; fp32 per vector, fp64 across vectors and lanes.
template <class E, bool kVec>
__device__ double resid_chunk_mass(const char* trow, const char* drow, int32_t c0, int32_t n, float k2,
                                   const ReqInfo& in, int lane) {
  double acc = 0.0;
  if constexpr (kVec) {
    const u32x4* tp = reinterpret_cast<const u32x4*>(trow + (int64_t)c0 * E::kBytes);
    const u32x4* dp = reinterpret_cast<const u32x4*>(drow + (int64_t)c0 * E::kBytes);
    const int32_t nvec = n / E::kPerVec;
#pragma unroll 4
    for (int k = 0; k < kVecPerLane; ++k) {
      const int vi = lane + kWave * k;
      if (vi < nvec) {
        float ft[E::kPerVec], fd[E::kPerVec];
        E::unpack(tp[vi], ft);
        E::unpack(dp[vi], fd);
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e) ft[e] = resid_weight(ft[e], fd[e], k2, in.ref_t, in.e_hi, in.e_lo);
        acc += (double)tree_sum(ft);
      }
    }
  } else {
    for (int32_t v = c0 + lane; v < c0 + n; v += kWave)
      acc += (double)resid_weight(E::at(trow, v), E::at(drow, v), k2, in.ref_t, in.e_hi, in.e_lo);
  }
  return wave_sum(acc);
}

// Inverse CDF inside one chunk: the smallest v with (mass of chunk elements up to v) > target.
// Each lane owns a contiguous run of the chunk; a wave scan of the run totals finds the lane and
// that lane walks its run.  If rounding leaves the target unreached, the last element of positive
// weight is taken.
template <class E>
__device__ int32_t search_chunk(bool residual, const char* trow, const char* drow, int32_t c0, int32_t n,
                                double target, float k2, const ReqInfo& in, int lane) {
  const int32_t run = (n + kWave - 1) / kWave;
  const int32_t b = min(c0 + lane * run, c0 + n);
  const int32_t e = min(b + run, c0 + n);
  auto weight = [&](int32_t v) -> float {
    return residual ? resid_weight(E::at(trow, v), E::at(drow, v), k2, in.ref_t, in.e_hi, in.e_lo)
                    : target_weight(E::at(trow, v), k2, in.ref_t);
  };
  double tot = 0.0;
  int32_t last_pos = -1;
  for (int32_t v = b; v < e; ++v) {
    const float w = weight(v);
    tot += (double)w;
    if (w > 0.0f) last_pos = v;
  }
  const double before = wave_exclusive_scan(tot, lane);
  const uint64_t hit = __ballot(b < e && before + tot > target);
  int32_t y = -1;
  if (hit) {
    const int f = __ffsll((unsigned long long)hit) - 1;
    if (lane == f) {
      double acc = before;
      y = last_pos;
      for (int32_t v = b; v < e; ++v) {
        acc += (double)weight(v);
        if (acc > target) {
          y = v;
          break;
        }
      }
    }
    y = __shfl(y, f, kWave);
  } else {
    const uint64_t has = __ballot(last_pos >= 0);
    if (has) {
      const int h = 63 - __clzll((long long)has);
      y = __shfl(last_pos, h, kWave);
    }
  }
  return y < 0 ? c0 + n - 1 : y;
}

template <class E, bool kVec>
__global__ __launch_bounds__(256) void terminal_draw(const void* __restrict__ target, const void* __restrict__ draft,
                                                     int32_t V, int32_t n_chunks, float k2,
                                                     const float2* __restrict__ part,
                                                     const ReqInfo* __restrict__ info,
                                                     int32_t* __restrict__ out_tokens, double* __restrict__ mass,
                                                     int32_t* __restrict__ diag_kind) {
  const int32_t i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const ReqInfo in = info[i];
  if (in.kind != SDV_TERM_BONUS && in.kind != SDV_TERM_RESIDUAL) return;  // uniform over the block
  double* m = mass + (int64_t)i * n_chunks;
  const char* trow = row_ptr<E>(target, in.trow, V);
  const char* drow = in.kind == SDV_TERM_RESIDUAL ? row_ptr<E>(draft, in.drow, V) : nullptr;
  if (in.kind == SDV_TERM_RESIDUAL) {
    for (int32_t c = wave; c < n_chunks; c += blockDim.x / kWave) {
      const int32_t c0 = c * E::kChunk;
      const double cm = resid_chunk_mass<E, kVec>(trow, drow, c0, min(E::kChunk, V - c0), k2, in, lane);
      if (lane == 0) m[c] = cm;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // lane 0 walks the chunk masses in ascending order
  const float2* tp = part + (int64_t)in.trow * n_chunks;
  bool residual = in.kind == SDV_TERM_RESIDUAL;
  int32_t cstar = 0;
  double target_in_chunk = 0.0;
  if (lane == 0) {
    double S = 0.0;
    if (residual) {
      for (int32_t c = 0; c < n_chunks; ++c) S += m[c];
      if (!(S > 0.0)) residual = false;  // no positive residual weight: fall back to p
    }
    if (!residual) {
      S = 0.0;
      for (int32_t c = 0; c < n_chunks; ++c) {
        m[c] = (double)tp[c].y * exp2((double)tp[c].x - (double)in.ref_t);
        S += m[c];
      }
    }
    const double U = (double)in.u * S;
    double below = 0.0;
    cstar = -1;
    for (int32_t c = 0; c < n_chunks; ++c) {
      if (below + m[c] > U) {
        cstar = c;
        break;
      }
      below += m[c];
    }
    if (cstar < 0) {  // rounding: the last chunk with positive mass
      below = 0.0;
      for (int32_t c = 0; c < n_chunks; ++c)
        if (m[c] > 0.0) cstar = c;
      if (cstar < 0) cstar = n_chunks - 1;
      for (int32_t c = 0; c < cstar; ++c) below += m[c];
    }
    target_in_chunk = U - below;
  }
  residual = __shfl((int)residual, 0, kWave) != 0;
  cstar = __shfl(cstar, 0, kWave);
  target_in_chunk = __shfl(target_in_chunk, 0, kWave);
  const int32_t c0 = cstar * E::kChunk;
  const int32_t y = search_chunk<E>(residual, trow, drow, c0, min(E::kChunk, V - c0), target_in_chunk, k2, in, lane);
  if (lane == 0) {
    out_tokens[in.trow] = y;
    if (diag_kind && in.kind == SDV_TERM_RESIDUAL && !residual) diag_kind[i] = SDV_TERM_RESIDUAL_EMPTY;
  }
}

// ============================================================================ Philox test hook

__global__ void philox_kernel(const uint32_t* __restrict__ ctr, const uint32_t* __restrict__ key, int64_t n,
                              uint32_t* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n) return;
  const Philox4 r = philox4x32_10(ctr[4 * b], ctr[4 * b + 1], ctr[4 * b + 2], ctr[4 * b + 3], key[2 * b], key[2 * b + 1]);
  out[4 * b] = r.w0;
  out[4 * b + 1] = r.w1;
  out[4 * b + 2] = r.w2;
  out[4 * b + 3] = r.w3;
}

// ============================================================================ host side

struct Layout {
  int32_t n_chunks;
  int64_t n_target_rows;
  size_t part_off, info_off, mass_off, total;
};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Returns SDV_OK and fills the layout, or the status the shape violates.
inline int make_layout(int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype, Layout* L) {
  if (dtype != SDV_BF16 && dtype != SDV_FP32) return SDV_ERR_UNSUPPORTED;
  if (B < 1 || n_draft_rows < 0 || V < 1) return SDV_ERR_INVALID_ARG;
  const int64_t n_t = n_draft_rows + B;
  const int64_t rows = n_t + n_draft_rows;
  if (rows > INT32_MAX) return SDV_ERR_LIMIT;
  const int32_t chunk = dtype == SDV_BF16 ? Bf16::kChunk : F32::kChunk;
  const int32_t n_chunks = (int32_t)((V + (int64_t)chunk - 1) / chunk);
  const int64_t units = rows * n_chunks;
  if ((units + 3) / 4 > INT32_MAX) return SDV_ERR_LIMIT;
  L->n_chunks = n_chunks;
  L->n_target_rows = n_t;
  L->part_off = 0;
  L->info_off = align_up((size_t)units * sizeof(float2));
  L->mass_off = L->info_off + align_up((size_t)B * sizeof(ReqInfo));
  L->total = L->mass_off + align_up((size_t)B * n_chunks * sizeof(double));
  return SDV_OK;
}

template <class E>
int launch_all(const void* target, const void* draft, const int32_t* tokens, const int32_t* cu, int32_t B,
               int64_t n_d, int32_t V, double T, uint64_t seed, int32_t* accepted_len, int32_t* out_tokens,
               char* ws, const Layout& L, hipStream_t stream, const sdv_diag* diag) {
  const bool greedy = T == 0.0;
  const float k2 = greedy ? 1.0f : (float)(1.4426950408889634074 / T);  // log2(e) / T
  const bool vec = ((uintptr_t)target % 16 == 0) && (draft == nullptr || (uintptr_t)draft % 16 == 0) &&
                   ((int64_t)V * E::kBytes) % 16 == 0;
  float2* part = reinterpret_cast<float2*>(ws + L.part_off);
  ReqInfo* info = reinterpret_cast<ReqInfo*>(ws + L.info_off);
  double* mass = reinterpret_cast<double*>(ws + L.mass_off);
  DiagPtrs dg{};
  if (diag) {
    dg = DiagPtrs{diag->target_lse, diag->draft_lse, diag->target_argmax, diag->ratio,
                  diag->accept_uniform, diag->draw_uniform, diag->terminal_kind};
  }
  auto record = [&](int k) {
    if (diag && diag->events[k]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(diag->events[k]), stream);
  };
  const int32_t n_t = (int32_t)L.n_target_rows;
  const int64_t rows = greedy ? n_t : n_t + n_d;
  const int64_t units = rows * L.n_chunks;
  const dim3 blk1(256);
  const dim3 grid1((unsigned)((units + 3) / 4));

  record(0);
  if (greedy) {
    if (vec)
      hipLaunchKernelGGL((row_pass_vec<E, true>), grid1, blk1, 0, stream, target, draft, n_t, V, L.n_chunks, units, k2, part);
    else
      hipLaunchKernelGGL((row_pass_scalar<E, true>), grid1, blk1, 0, stream, target, draft, n_t, V, L.n_chunks, units, k2, part);
  } else {
    if (vec)
      hipLaunchKernelGGL((row_pass_vec<E, false>), grid1, blk1, 0, stream, target, draft, n_t, V, L.n_chunks, units, k2, part);
    else
      hipLaunchKernelGGL((row_pass_scalar<E, false>), grid1, blk1, 0, stream, target, draft, n_t, V, L.n_chunks, units, k2, part);
  }
  if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
  record(1);
  if (greedy)
    hipLaunchKernelGGL((accept_scan<E, true>), dim3(B), dim3(kWave), 0, stream, target, draft, tokens, cu, B,
                       (int32_t)n_d, V, L.n_chunks, k2, seed, part, accepted_len, out_tokens, info, dg);
  else
    hipLaunchKernelGGL((accept_scan<E, false>), dim3(B), dim3(kWave), 0, stream, target, draft, tokens, cu, B,
                       (int32_t)n_d, V, L.n_chunks, k2, seed, part, accepted_len, out_tokens, info, dg);
  if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
  record(2);
  if (!greedy) {
    if (vec)
      hipLaunchKernelGGL((terminal_draw<E, true>), dim3(B), dim3(256), 0, stream, target, draft, V, L.n_chunks, k2, part,
                         info, out_tokens, mass, dg.terminal_kind);
    else
      hipLaunchKernelGGL((terminal_draw<E, false>), dim3(B), dim3(256), 0, stream, target, draft, V, L.n_chunks, k2, part,
                         info, out_tokens, mass, dg.terminal_kind);
    if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
    record(3);
  }
  return SDV_OK;
}

}  // namespace sdv

extern "C" {

size_t sdv_workspace_bytes(int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype) {
  sdv::Layout L;
  return sdv::make_layout(B, n_draft_rows, V, dtype, &L) == SDV_OK ? L.total : 0;
}

int sdv_verify_ex(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                  const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                  double temperature, uint64_t seed, int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                  size_t workspace_bytes, void* stream, const sdv_diag* diag) {
  sdv::Layout L;
  const int shape = sdv::make_layout(B, n_draft_rows, V, dtype, &L);
  if (shape != SDV_OK) return shape;
  if (!target_logits || !ragged_offsets || !accepted_len || !out_tokens) return SDV_ERR_INVALID_ARG;
  if (n_draft_rows > 0 && !draft_tokens) return SDV_ERR_INVALID_ARG;
  if (!(temperature >= 0.0) || !isfinite(temperature)) return SDV_ERR_INVALID_ARG;
  if (temperature > 0.0) {
    const double k2 = 1.4426950408889634074 / temperature;
    if (!isfinite((float)k2)) return SDV_ERR_INVALID_ARG;
    if (n_draft_rows > 0 && !draft_logits) return SDV_ERR_INVALID_ARG;
  }
  if (!workspace || workspace_bytes < L.total || (uintptr_t)workspace % sdv::kAlign != 0) return SDV_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (dtype == SDV_BF16)
    return sdv::launch_all<sdv::Bf16>(target_logits, draft_logits, draft_tokens, ragged_offsets, B, n_draft_rows, V,
                                      temperature, seed, accepted_len, out_tokens, ws, L, s, diag);
  return sdv::launch_all<sdv::F32>(target_logits, draft_logits, draft_tokens, ragged_offsets, B, n_draft_rows, V,
                                   temperature, seed, accepted_len, out_tokens, ws, L, s, diag);
}

int sdv_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
               const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
               double temperature, uint64_t seed, int32_t* accepted_len, int32_t* out_tokens, void* workspace,
               size_t workspace_bytes, void* stream) {
  return sdv_verify_ex(target_logits, draft_logits, draft_tokens, ragged_offsets, B, n_draft_rows, V, dtype,
                       temperature, seed, accepted_len, out_tokens, workspace, workspace_bytes, stream, nullptr);
}

int sdv_philox4x32_10(const uint32_t* counters, const uint32_t* keys, int64_t n, uint32_t* out, void* stream) {
  if (!counters || !keys || !out || n < 1) return SDV_ERR_INVALID_ARG;
  if ((n + 255) / 256 > INT32_MAX) return SDV_ERR_LIMIT;
  hipLaunchKernelGGL(sdv::philox_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), counters, keys, n, out);
  return hipGetLastError() == hipSuccess ? SDV_OK : SDV_ERR_HIP;
}

const char* sdv_status_string(int status) {
  switch (status) {
    case SDV_OK: return "ok";
    case SDV_ERR_INVALID_ARG: return "invalid argument";
    case SDV_ERR_UNSUPPORTED: return "unsupported dtype";
    case SDV_ERR_LIMIT: return "batch exceeds a size limit";
    case SDV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SDV_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

int sdv_abi_version(void) { return SDV_ABI_VERSION; }

}  // extern "C"
