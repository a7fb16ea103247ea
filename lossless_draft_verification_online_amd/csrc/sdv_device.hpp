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
// xor butterflies: at every level both partners add the same two values, so every lane ends with
// the bit-identical result.

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Larger value wins; equal values go to the smaller index.
__device__ __forceinline__ void wave_argmax(float& v, int32_t& idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int32_t oi = __shfl_xor(idx, o, kWave);
    if (ov > v || (ov == v && oi < idx)) {
      v = ov;
      idx = oi;
    }
  }
}

// Exclusive prefix sum over the wave (lane order), fp64.
__device__ __forceinline__ double wave_exclusive_scan(double v, int lane) {
  double incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double up = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += up;
  }
  return incl - v;
}

// Sum of the eight (or four) elements of one vector as a balanced tree.
template <int N>
__device__ __forceinline__ float tree_sum(const float (&f)[N]) {
  if constexpr (N == 8) {
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
