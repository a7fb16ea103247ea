// Device helpers for the gfx950 verification kernels: logit element formats, 16-byte vector
// loads, wave64 reductions and the verifier's Philox4x32-10 stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdv {

constexpr int kWave = 64;
// One work unit of the row pass streams 16 KiB of one row: 16 vectors of 16 bytes per lane.
constexpr int kChunkBytes = 16384;
constexpr int kVecPerLane = kChunkBytes / (16 * kWave);

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------- element formats

struct Bf16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  static constexpr int kChunk = kChunkBytes / kBytes;
  // bf16 is the upper half of a binary32: the even element sits in the low 16 bits of a word.
  __device__ static __forceinline__ void unpack(const u32x4 v, float (&f)[kPerVec]) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static __forceinline__ float at(const void* row, int64_t v) {
    return __uint_as_float((uint32_t)(static_cast<const uint16_t*>(row)[v]) << 16);
  }
  static constexpr uint32_t kNegInfWord = 0xff80ff80u;  // two bf16 -inf
};

struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
  static constexpr int kChunk = kChunkBytes / kBytes;
  __device__ static __forceinline__ void unpack(const u32x4 v, float (&f)[kPerVec]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ float at(const void* row, int64_t v) { return static_cast<const float*>(row)[v]; }
  static constexpr uint32_t kNegInfWord = 0xff800000u;
};

template <class E>
__device__ __forceinline__ const char* row_ptr(const void* base, int64_t row, int32_t V) {
  return static_cast<const char*>(base) + row * (int64_t)V * E::kBytes;
}

// ----------------------------------------------------------------------------- wave64 reductions
// Butterflies with every lane of the wave active.  Inside a row of 16 lanes the partner comes by a
// DPP move: lane ^ 1 and lane ^ 2 (quad permutes), then the mirror inside 8 lanes and inside 16
// (after the quad steps each quad holds one value, so a mirror combines whole quads, then whole
// halves).  Across rows the gfx950 row swaps hand every lane both rows' values: rows 2r and 2r + 1
// (permlane16 swap), then the two halves of the wave (permlane32 swap).  Both partners combine the
// same two operands with a commutative operation, so every lane ends with the bit-identical result.
// Scans use DPP row shifts by 1, 2, 4, 8, then the row broadcasts of lanes 15 and 31.

namespace wave_detail {
constexpr int kXor1 = 0xb1, kXor2 = 0x4e, kHalfMirror = 0x141, kMirror = 0x140, kRowShr = 0x110, kBcast15 = 0x142,
              kBcast31 = 0x143;
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {  // lanes the control leaves without a source read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xf, false);
}
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ float dpp(float v) {
  return __uint_as_float(dpp<kCtrl, kRowMask>(__float_as_uint(v)));
}
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ uint64_t dpp(uint64_t v) {
  const uint64_t lo = dpp<kCtrl, kRowMask>((uint32_t)v), hi = dpp<kCtrl, kRowMask>((uint32_t)(v >> 32));
  return (hi << 32) | lo;
}
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ double dpp(double v) {
  return __longlong_as_double((long long)dpp<kCtrl, kRowMask>((uint64_t)__double_as_longlong(v)));
}
// Both rows' (or halves') values of a 32-bit word: lower in lo, upper in hi, in every lane.
template <int kSpan>
__device__ __forceinline__ void both(uint32_t v, uint32_t& lo, uint32_t& hi) {
  if constexpr (kSpan == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    lo = r[0];
    hi = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    lo = r[0];
    hi = r[1];
  }
}
template <int kSpan>
__device__ __forceinline__ void both(uint64_t v, uint64_t& lo, uint64_t& hi) {
  uint32_t l0, l1, h0, h1;
  both<kSpan>((uint32_t)v, l0, l1);
  both<kSpan>((uint32_t)(v >> 32), h0, h1);
  lo = ((uint64_t)h0 << 32) | l0;
  hi = ((uint64_t)h1 << 32) | l1;
}
template <int kSpan>
__device__ __forceinline__ void both(float v, float& lo, float& hi) {
  uint32_t a, b;
  both<kSpan>(__float_as_uint(v), a, b);
  lo = __uint_as_float(a);
  hi = __uint_as_float(b);
}
template <int kSpan>
__device__ __forceinline__ void both(double v, double& lo, double& hi) {
  uint64_t a, b;
  both<kSpan>((uint64_t)__double_as_longlong(v), a, b);
  lo = __longlong_as_double((long long)a);
  hi = __longlong_as_double((long long)b);
}
// The same combine within each row of 16 lanes: every lane ends with its row's value.
template <class T, class Op>
__device__ __forceinline__ T row_reduce(T v, Op op) {
  v = op(v, dpp<kXor1>(v));
  v = op(v, dpp<kXor2>(v));
  v = op(v, dpp<kHalfMirror>(v));
  return op(v, dpp<kMirror>(v));
}
// The same combine within each half wave (32 lanes).
template <class T, class Op>
__device__ __forceinline__ T half_reduce(T v, Op op) {
  v = row_reduce(v, op);
  T lo, hi;
  both<16>(v, lo, hi);
  return op(lo, hi);
}
// An all-reduce with a commutative combine (binary32, binary64, 32- or 64-bit unsigned): the rows
// of 16 lanes first, then the half waves, then across them.
template <class T, class Op>
__device__ __forceinline__ T all_reduce(T v, Op op) {
  v = half_reduce(v, op);
  T lo, hi;
  both<32>(v, lo, hi);
  return op(lo, hi);
}
// Inclusive prefix sum in lane order.
template <class T>
__device__ __forceinline__ T inclusive_scan(T v) {
  v += dpp<kRowShr + 1>(v);
  v += dpp<kRowShr + 2>(v);
  v += dpp<kRowShr + 4>(v);
  v += dpp<kRowShr + 8>(v);
  v += dpp<kBcast15, 0xa>(v);
  v += dpp<kBcast31, 0xc>(v);
  return v;
}
}  // namespace wave_detail

__device__ __forceinline__ float wave_max(float v) {
  return wave_detail::all_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_detail::all_reduce(v, [](float a, float b) { return a + b; });
}

__device__ __forceinline__ double wave_sum(double v) {
  return wave_detail::all_reduce(v, [](double a, double b) { return a + b; });
}

// Per row of 16 lanes.
__device__ __forceinline__ float row16_max(float v) {
  return wave_detail::row_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ double row16_sum(double v) {
  return wave_detail::row_reduce(v, [](double a, double b) { return a + b; });
}

// Per half wave (32 lanes).
__device__ __forceinline__ float half_max(float v) {
  return wave_detail::half_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ double half_sum(double v) {
  return wave_detail::half_reduce(v, [](double a, double b) { return a + b; });
}

// Larger value wins; equal values go to the smaller index.
__device__ __forceinline__ void wave_argmax(float& v, int32_t& idx) {
  using namespace wave_detail;
  auto take = [&](float ov, int32_t oi) {
    if (ov > v || (ov == v && oi < idx)) {
      v = ov;
      idx = oi;
    }
  };
  take(__uint_as_float(dpp<kXor1>(__float_as_uint(v))), (int32_t)dpp<kXor1>((uint32_t)idx));
  take(__uint_as_float(dpp<kXor2>(__float_as_uint(v))), (int32_t)dpp<kXor2>((uint32_t)idx));
  take(__uint_as_float(dpp<kHalfMirror>(__float_as_uint(v))), (int32_t)dpp<kHalfMirror>((uint32_t)idx));
  take(__uint_as_float(dpp<kMirror>(__float_as_uint(v))), (int32_t)dpp<kMirror>((uint32_t)idx));
  uint32_t va, vb, ia, ib;
  both<16>(__float_as_uint(v), va, vb);
  both<16>((uint32_t)idx, ia, ib);
  v = __uint_as_float(va);
  idx = (int32_t)ia;
  take(__uint_as_float(vb), (int32_t)ib);
  both<32>(__float_as_uint(v), va, vb);
  both<32>((uint32_t)idx, ia, ib);
  v = __uint_as_float(va);
  idx = (int32_t)ia;
  take(__uint_as_float(vb), (int32_t)ib);
}

// Exclusive prefix sum over the wave (lane order), fp64: the inclusive scan less the lane's value.
__device__ __forceinline__ double wave_exclusive_scan(double v, int) {
  return wave_detail::inclusive_scan(v) - v;
}

// Inclusive prefix sums over the wave (lane order) of 32- and 64-bit unsigned integers.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) { return wave_detail::inclusive_scan(v); }
__device__ __forceinline__ uint64_t wave_inclusive_scan(uint64_t v) { return wave_detail::inclusive_scan(v); }

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return wave_detail::all_reduce(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  return wave_detail::all_reduce(v, [](uint64_t a, uint64_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_detail::all_reduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

// The value of lane src (the same index in every lane) in every lane.
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int src) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, src);
}
__device__ __forceinline__ int32_t lane_value(int32_t v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ uint64_t lane_value(uint64_t v, int src) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), src) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
}
__device__ __forceinline__ double lane_value(double v, int src) {
  return __longlong_as_double((long long)lane_value((uint64_t)__double_as_longlong(v), src));
}

// Sum of 4, 8 or 16 values as a balanced tree.
template <int N>
__device__ __forceinline__ float tree_sum(const float (&f)[N]) {
  static_assert(N == 4 || N == 8 || N == 16, "pairwise sums of 4, 8 or 16 values");
  if constexpr (N == 16) {
    return (((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]))) +
           (((f[8] + f[9]) + (f[10] + f[11])) + ((f[12] + f[13]) + (f[14] + f[15])));
  } else if constexpr (N == 8) {
    return ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
  } else {
    return (f[0] + f[1]) + (f[2] + f[3]);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): ten
// rounds; each multiplies counter words 0 and 2 by the round constants, folds the high product
// halves into words 1 and 3 together with the key, and the key advances by the Weyl increments
// after every round.

struct Philox4 {
  uint32_t w0, w1, w2, w3;
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                        uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint32_t hi_a = __umulhi(0xD2511F53u, c0), lo_a = 0xD2511F53u * c0;
    const uint32_t hi_b = __umulhi(0xCD9E8D57u, c2), lo_b = 0xCD9E8D57u * c2;
    c0 = hi_b ^ c1 ^ k0;
    c1 = lo_b;
    c2 = hi_a ^ c3 ^ k1;
    c3 = lo_a;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// The verifier's block for (request, position): key = seed, counter = (position, request, 0, 0).
__device__ __forceinline__ Philox4 verifier_block(uint64_t seed, uint32_t request, uint32_t position) {
  return philox4x32_10(position, request, 0u, 0u, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// Accept-test uniform in (0, 1] from word 0 and draw uniform in [0, 1) from word 1, both exact in fp32.
__device__ __forceinline__ float accept_uniform(const Philox4& b) { return (float)((b.w0 >> 8) + 1u) * 0x1.0p-24f; }
__device__ __forceinline__ float draw_uniform(const Philox4& b) { return (float)(b.w1 >> 8) * 0x1.0p-24f; }

}  // namespace sdv
