// Batched speculative-sampling verification on MI355X (gfx950): kernels and the C ABI.
//
// The step verifies every request of a ragged batch at once (SDCP "Verification and Commit",
// steps 5 to 7; Rule 1 and Rule 2 of its section "Acceptance Rules"; the r <= p/q test of
// "SOTA-227", section "What to do").  Two kernels run on the caller's stream (two more between
// them when a call carries top-k / top-p, section 2):
//
//  row_records   The stream.  One wave64 per 16 KiB chunk of every logit row reads the chunk once
//                with 16-byte loads.  At T > 0 it records the chunk's exponent reference
//                ref = fl(max z * k) and s = sum 2^(z k - ref), k = log2(e)/T; at T = 0 the chunk's
//                maximum and the smallest index reaching it.  Waves never wait on each other, so
//                nothing interrupts the stream.  In a top-k / top-p call on bf16 rows it also counts
//                the logits of the 128 keys at and below each chunk's maximum.
//  verdicts      One workgroup of 8 waves per request.  The waves fold the request's rows from
//                their chunk records (fp64, lanes over chunks) into shared memory; wave 0 gathers the
//                target and draft logits at each draft token, forms p/q, draws r from Philox
//                (seed; position, request), and a ballot finds the first rejection.  Greedy
//                terminals come from the folded argmax.  A bonus is drawn from p at position K
//                using the bonus row's chunk records and one chunk re-read; a correction needs the
//                chunk masses of max(p - q, 0) on the rejected row pair, which the 8 waves compute
//                into shared memory before wave 0 draws.  A batch too small to occupy the compute
//                units gets several workgroups per request, which share that pass (section 3).
//  tree_verdicts Token trees (section 4), in place of verdicts: one workgroup of 16 waves per
//                request walks its tree in wave 0, and the whole workgroup computes the residual
//                masses after each rejected child.
//
// Rows that are not 16-byte aligned (an odd vocabulary, a base on an element boundary) take the
// same 16-byte loads: each chunk is split at 16-byte boundaries, the few elements before the first
// vector and after the last go one per lane, and a second row of a pair is realigned to the first
// by one shift (section "rows off the 16-byte grid").
//
// The kernel boundary orders the stream before the verdicts.  Inside a kernel only the verdict
// workgroups of one request hand anything over: a correction's chunk masses, through the
// workspace, behind a device-scope fence and a counter; no workgroup ever waits for another.  No
// matrix cores are involved: nothing here is a contraction, and the roofline is HBM bandwidth.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

#include "../../include/sdv.h"
#include "sdv_device.hpp"
#include "split.hpp"

namespace sdv {

constexpr double kLn2 = 0.69314718055994530942;

struct DiagPtrs {
  double* target_lse;
  double* draft_lse;
  int32_t* target_argmax;
  double* ratio;
  float* accept_uniform;
  float* draw_uniform;
  int32_t* terminal_kind;
  float* target_logit;
  float* draft_logit;
  double* terminal_mass;
};

constexpr int32_t kMaxChunks = 4096;  // chunks per row: the verdict and cut kernels keep one value per chunk in LDS
constexpr int kVerdictWaves = 8;      // waves of a verdict workgroup
constexpr int kWideVerdictWaves = 16; // waves of a verdict workgroup for small batches of short rows

// Truncating bf16 calls: the row pass also counts, per chunk, the logits of each of the kHistKeys
// 16-bit order keys at and below the chunk maximum's (one binade of positive logits), so that a cut
// among the largest logits needs no second read of the row.  The chunk's top key carries kNoCounts
// when its window would reach zero or -inf (then its counts are all zero).
constexpr int kHistKeys = 128;
constexpr uint32_t kNoCounts = 0x10000u;
constexpr uint32_t kCountNothing = 0x40000000u;  // a stand-in maximum more than kHistKeys + 63 above every 16-bit pattern

// Order keys of bf16 logits: a larger logit has a larger key and -0 shares the key of +0.
// The 16-bit key of a bf16 logit (its raw bits h), and the 32-bit key of a 16-bit one: below the
// 16 bits a bf16 key holds 16 copies of its sign bit's complement.
__device__ __forceinline__ uint32_t key16_of_bits(uint32_t h) {
  h = h == 0x8000u ? 0u : h;
  return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
}
__device__ __forceinline__ uint32_t key16_to_key(uint32_t key) {
  return (key << 16) | ((key & 0x8000u) ? 0u : 0xffffu);
}

// The tokens a truncated row keeps (top-k / top-p) are its leading ranks in the order "larger logit
// first, smaller id first among equal logits", so the last kept rank describes them: token v is
// kept iff z_v > kappa, or z_v == kappa and v <= vcut.  A row that is not truncated has
// kappa = -inf and vcut = INT32_MAX.
struct Cut {
  float kappa;
  int32_t vcut;
};

__device__ __forceinline__ bool kept_by(const Cut c, float z, int32_t v) {
  return z > c.kappa || (z == c.kappa && v <= c.vcut);
}

// The smallest binary32 value above kappa (NaN above +inf, so that nothing lies above it): z > kappa
// iff z >= above(kappa) for every z.
__device__ __forceinline__ float above(float kappa) {
  const uint32_t b = __float_as_uint(kappa);
  if (kappa == INFINITY) return __builtin_nanf("");
  if ((b & 0x7fffffffu) == 0u) return __uint_as_float(1u);  // +-0: the smallest subnormal
  return __uint_as_float((b & 0x80000000u) ? b - 1u : b + 1u);
}

// The tokens the rows of a terminal draw keep: NoCut keeps every token (its tests fold away),
// RowCuts holds the cuts of the target row (t) and of the draft row (d), each as a threshold on the
// logit that depends on the token id: kappa up to vcut, the next value above kappa after it (the
// same test as kept_by, one compare on the logit and one on the id).
struct NoCut {
  __device__ __forceinline__ bool t(float, int32_t) const { return true; }
  __device__ __forceinline__ bool d(float, int32_t) const { return true; }
};
struct RowCuts {
  Cut ct, cd;
  float t_up, d_up;
  __device__ __forceinline__ RowCuts() : ct{-INFINITY, INT32_MAX}, cd{-INFINITY, INT32_MAX}, t_up(-INFINITY), d_up(-INFINITY) {}
  __device__ __forceinline__ RowCuts(Cut t_cut, Cut d_cut)
      : ct(t_cut), cd(d_cut), t_up(above(t_cut.kappa)), d_up(above(d_cut.kappa)) {}
  __device__ __forceinline__ bool t(float z, int32_t v) const { return z >= (v <= ct.vcut ? ct.kappa : t_up); }
  __device__ __forceinline__ bool d(float z, int32_t v) const { return z >= (v <= cd.vcut ? cd.kappa : d_up); }
};

struct Params {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* cu;
  int32_t* accepted_len;
  int32_t* out_tokens;
  float2* part;         // [row slots][Cs] chunk records; target row r is slot r, draft row d slot n_t + d
  int32_t B, n_d, n_t, V, C;
  int64_t n_units;
  int64_t lds_records;  // chunk records the verdict kernel can stage in shared memory
  float k2;  // log2(e) / T, or 0 for the greedy rule (one profile for the whole batch)
  uint64_t seed;
  const float* temp_each;     // [B] temperature of each request, or null: one profile for the batch
  const uint64_t* seed_each;  // [B] seed of each request (with temp_each)
  const double* r_each;       // [n_d] caller's accept uniforms in [0, 1), or null: Philox
  const double* u_each;       // [n_t] caller's draw uniforms in [0, 1) per position (with r_each)
  const int32_t* stop_off;    // [B + 1] stop-token lists (CSR into stop_tok), or null
  const int32_t* stop_tok;    // [n_stop]
  int64_t n_stop;
  const int32_t* budget;      // [B] remaining output tokens, or null: no limit
  int32_t* emitted_len;       // [B] out: tokens emitted after truncation, or null
  const float* qrows;         // [n_d][V] draft distributions (binary32) in place of draft logits, or null
  const int32_t* top_k;       // [B] top-k of each request's profile, or null (0: none)
  const int32_t* top_p_milli; // [B] top-p in thousandths, or null (1000: none)
  int32_t* kept_tokens;       // [row slots] out: tokens each truncated row keeps, or null
  Cut* cuts;                  // [row slots] the cut of every row (workspace), read when truncation is on
  uint32_t* hist;             // [row slots][C][kHistKeys / 2] per-chunk key counts, two 16-bit counts a word
  uint32_t* hist_top;         // [row slots][C] the chunk maximum's key, | kNoCounts without counts
  int32_t* pending;           // [1 + row slots] rows the count kernel leaves to row_cuts: count, then slots
  int32_t split;              // verdict workgroups per request (split > 1: the residual pass is shared)
  double* split_mass;         // [B][Cm] residual chunk masses of a request's correction, published by the waves or
                              // workgroups that compute them (each request's on 128-byte lines of their own)
  uint32_t* split_count;      // [B][kLineWords] masses published per request (zeroed by the row pass), a line each
  int32_t Cm;                 // C rounded up to 16: a request's masses fill whole 128-byte lines
  int32_t* batch_ok;          // [1] the offsets are valid (written by the row pass's first workgroup)
  const int32_t* parents;     // [n_d] token trees: each node's parent within its request (-1: the root), or null
  const int32_t* draft_row;   // [n_d] token trees: each node's draft row, or null (node d: row d)
  int32_t n_dr;               // token trees: draft rows given (and streamed)
  int32_t* accepted_nodes;    // [n_d] token trees, out: the accepted path's nodes, then -1
  DiagPtrs dg;
};

// ============================================================================ sampling profiles

// k = log2(e) / T in fp32 for a temperature T: 0 selects the greedy rule; NaN marks a temperature
// that describes no profile (negative, NaN, infinite, or so small that k overflows fp32).
__device__ __forceinline__ float k2_of(float T) {
  if (T == 0.0f) return 0.0f;
  if (!(T > 0.0f) || isinf(T)) return __int_as_float(0x7fc00000);
  const float k2 = (float)(1.4426950408889634074 / (double)T);
  return isfinite(k2) && k2 > 0.0f ? k2 : __int_as_float(0x7fc00000);
}

// The request a logit row belongs to, by a wave-uniform binary search over the offsets read through
// the scalar cache (these reads do not wait behind the stream's vector loads).  Target row r
// belongs to the largest i < B with cu[i] + i <= r; draft row d to the largest i < B with
// cu[i] <= d.  Offsets that are not non-decreasing still give an index in [0, B); such batches are
// rejected by the verdict kernel.
__device__ __forceinline__ int32_t request_of_row(const int32_t* cu, int32_t B, int32_t row, bool target) {
  const __attribute__((address_space(4))) int32_t* c = (const __attribute__((address_space(4))) int32_t*)cu;
  int32_t lo = 0, hi = B;
  while (hi - lo > 1) {
    const int32_t mid = lo + (hi - lo) / 2;
    const int64_t key = (int64_t)c[mid] + (target ? mid : 0);
    if (key <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

// The same lookup by a whole wave (every lane active): lanes test 64 evenly spaced requests, and
// the last one whose first row is at or before row narrows the range to one lane's share; the
// first rows are non-decreasing in i, so the lanes that pass form a prefix.
__device__ __forceinline__ int32_t request_of_row_wave(const int32_t* cu, int32_t B, int32_t row, bool target,
                                                       int lane) {
  int32_t lo = 0, span = B;  // the request lies in [lo, lo + span)
  while (span > 1) {
    const int32_t step = (span + kWave - 1) / kWave;
    const int32_t i = lo + lane * step;
    const bool at_or_before = i < lo + span && (int64_t)cu[i] + (target ? i : 0) <= row;
    const uint64_t pass = __ballot(at_or_before);
    const int32_t last = pass ? 63 - __clzll((long long)pass) : 0;
    lo += last * step;
    span = min(step, span - last * step);
  }
  return lo;
}

// ============================================================================ offsets

// cu[0] = 0, non-decreasing, cu[B] = n_d.  Anything else rejects the whole batch.  One wave of the row
// pass checks this once per call and writes the answer for the verdict kernels.
__device__ __forceinline__ void screen_offsets(const Params& P, int lane) {
  bool bad = false;
  for (int32_t j = lane; j < P.B; j += kWave) bad |= P.cu[j] > P.cu[j + 1];
  if (lane == 0) bad |= P.cu[0] != 0 || P.cu[P.B] != P.n_d;
  const bool ok = __ballot(bad) == 0;
  if (lane == 0) *P.batch_ok = ok ? 1 : 0;
}

// Counters that waves on different compute units add to sit one to a 128-byte line: the atomic unit
// takes a line at a time, so counters sharing a line queue behind each other (measured on MI355X: a
// stream that counted 36 units on each of 32 counters packed in a line ran 38% slower than one with a
// counter per line).
constexpr int kLineWords = 32;

// ============================================================================ 1. the stream

template <class E>
__device__ __forceinline__ u32x4 neg_inf_vec() {
  return u32x4{E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord};
}

// Vector vi of a chunk with nvec vectors, -inf past the chunk's end.
template <class E>
__device__ __forceinline__ u32x4 load_vec(const u32x4* v, int vi, int32_t nvec) {
  return vi < nvec ? v[vi] : neg_inf_vec<E>();
}
template <class E>
__device__ __forceinline__ u32x4 load_vec_nt(const u32x4* v, int vi, int32_t nvec) {
  return vi < nvec ? __builtin_nontemporal_load(v + vi) : neg_inf_vec<E>();
}

// The 16 vectors per lane of one 16 KiB chunk (16-byte aligned rows), -inf past the row's end.
// The stream is read once: non-temporal loads keep it from displacing reused lines in L2.
template <class E>
__device__ __forceinline__ void load_chunk(const char* rp, int32_t c0, int32_t n, int lane, u32x4 (&buf)[kVecPerLane]) {
  const u32x4* vp = reinterpret_cast<const u32x4*>(rp + (int64_t)c0 * E::kBytes);
  const int32_t nvec = n / E::kPerVec;
#pragma unroll
  for (int k = 0; k < kVecPerLane; ++k) buf[k] = load_vec_nt<E>(vp, lane + kWave * k, nvec);
}

// The same 16 vectors per lane, moved by direct-to-LDS loads into the wave's 16 KiB slice `lds` and
// read back (a read yardstick's shape; vectors past the row's end are not loaded and read as -inf).
constexpr int kCpolNt = 2;  // cache-policy bits of a non-temporal load
template <class E>
__device__ __forceinline__ void load_chunk_lds(const char* rp, int32_t c0, int32_t n, int lane, u32x4* lds,
                                               u32x4 (&buf)[kVecPerLane]) {
  const u32x4* vp = reinterpret_cast<const u32x4*>(rp + (int64_t)c0 * E::kBytes);
  const int32_t nvec = n / E::kPerVec;
  typedef __attribute__((address_space(3))) void* lds_ptr;
#pragma unroll
  for (int k = 0; k < kVecPerLane; ++k)
    if (lane + kWave * k < nvec)
      __builtin_amdgcn_global_load_lds(vp + lane + kWave * k, (lds_ptr)(lds + kWave * k), 16, 0, kCpolNt);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int k = 0; k < kVecPerLane; ++k) buf[k] = lane + kWave * k < nvec ? lds[lane + kWave * k] : neg_inf_vec<E>();
}

// The maximum of a loaded chunk (every lane holds it).
template <class E>
__device__ __forceinline__ float chunk_max(u32x4 (&buf)[kVecPerLane]) {
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kVecPerLane; ++k) {
    float f[E::kPerVec];
    E::unpack(buf[k], f);
#pragma unroll
    for (int e = 0; e < E::kPerVec; ++e) m = fmaxf(m, f[e]);
  }
  return wave_max(m);
}

// sum 2^(z k - ref) over a loaded chunk.  kCount (bf16 only) also counts every logit into the
// wave's counters h: at d = hm - bits(z) (raw bf16 bits, unsigned arithmetic) when d < kHistKeys,
// else at the lane's spare counter `spare` (kHistKeys + lane, never read).  For a positive hm that
// selects exactly the kHistKeys keys at and below hm; negative logits, -0, the -inf padding and
// NaN wrap to a large d.  hm = kCountNothing sends every logit to the spare counter.  Every logit
// takes the same unmasked shared-memory add: no compare, no exec-mask change per logit.
template <class E, bool kCount>
__device__ __forceinline__ float exp_sum(u32x4 (&buf)[kVecPerLane], float k2, float ref, uint32_t hm,
                                         uint32_t spare, uint32_t* h) {
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t one = 1u;
  if constexpr (kCount) asm volatile("" : "+v"(one));  // held in a register, not rematerialized per add
#pragma unroll
  for (int k = 0; k < kVecPerLane; ++k) {
    // re-unpack from the raw words rather than keep every unpacked element live across the max
    asm volatile("" : "+v"(buf[k]));
    if constexpr (kCount) {
      const uint32_t wd[4] = {buf[k].x, buf[k].y, buf[k].z, buf[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t d_lo = hm - (wd[j] & 0xffffu), d_hi = hm - (wd[j] >> 16);
        atomicAdd(&h[d_lo < spare ? d_lo : spare], one);
        atomicAdd(&h[d_hi < spare ? d_hi : spare], one);
      }
    }
    float f[E::kPerVec];
    E::unpack(buf[k], f);
#pragma unroll
    for (int e = 0; e < E::kPerVec; ++e) f[e] = fast_exp2(fmaf(f[e], k2, -ref));
    acc[k & 3] += tree_sum(f);
  }
  return wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
}

// The record of a loaded chunk: (ref, sum 2^(z k - ref)) at T > 0, (max, first index of max) at T = 0.
template <class E, bool kGreedy>
__device__ __forceinline__ float2 record_of(u32x4 (&buf)[kVecPerLane], int32_t c0, float k2, int lane) {
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
    wave_argmax(best, idx);
    return make_float2(best, __int_as_float(idx));
  } else {
    const float m = chunk_max<E>(buf);
    if (m == -INFINITY) return make_float2(-INFINITY, 0.0f);
    const float ref = m * k2;
    return make_float2(ref, exp_sum<E, false>(buf, k2, ref, 0u, 0u, nullptr));
  }
}

// A chunk [c0, c0 + n) of a row that is only element-aligned, split at 16-byte boundaries: the
// aligned vectors inside it (from element c0 + head on) are loaded like an aligned row's, and the
// at most kPerVec - 1 elements before the first of them and after the last, one per lane (lanes
// [0, head) take the head, the next lanes the tail).  Every load stays inside the chunk.
struct SplitEdge {
  int32_t head;  // elements before the first aligned vector
  int32_t body;  // aligned vectors
  bool ok;       // the lane holds an edge element
  float z;       // the lane's edge element, -inf on lanes without one
  int32_t v;     // its index in the row
};
template <class E>
__device__ __forceinline__ SplitEdge load_split_chunk(const char* rp, int32_t c0, int32_t n, int lane,
                                                      u32x4 (&buf)[kVecPerLane]) {
  const split::Plan p = split::row((uintptr_t)rp, E::kBytes, c0, n);
  load_chunk<E>(rp, c0 + p.head, p.body * E::kPerVec, lane, buf);
  const int32_t e = split::edge(p.head, p.body * E::kPerVec, n, lane);
  SplitEdge s;
  s.head = p.head;
  s.body = p.body;
  s.ok = e >= 0;
  s.v = c0 + (s.ok ? e : 0);
  s.z = s.ok ? E::at(rp, s.v) : -INFINITY;
  return s;
}

// The record of a split chunk (as record_of: the vectors' elements plus the lane's edge element).
template <class E, bool kGreedy>
__device__ __forceinline__ float2 record_of_split(u32x4 (&buf)[kVecPerLane], const SplitEdge& s, int32_t c0, float k2,
                                                  int lane) {
  if constexpr (kGreedy) {
    float best = -INFINITY;
    int32_t idx = INT32_MAX;
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) {
      float f[E::kPerVec];
      E::unpack(buf[k], f);
      const int32_t e0 = c0 + s.head + (lane + kWave * k) * E::kPerVec;
#pragma unroll
      for (int e = 0; e < E::kPerVec; ++e) {
        if (f[e] > best) {
          best = f[e];
          idx = e0 + e;
        }
      }
    }
    // the edge element may precede the vectors: equal values go to the smaller index
    if (s.z > best || (s.z == best && s.z != -INFINITY && s.v < idx)) {
      best = s.z;
      idx = s.v;
    }
    wave_argmax(best, idx);
    return make_float2(best, __int_as_float(idx));
  } else {
    float m = s.z;
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) {
      float f[E::kPerVec];
      E::unpack(buf[k], f);
#pragma unroll
      for (int e = 0; e < E::kPerVec; ++e) m = fmaxf(m, f[e]);
    }
    m = wave_max(m);
    if (m == -INFINITY) return make_float2(-INFINITY, 0.0f);
    const float ref = m * k2;
    float acc[4] = {fast_exp2(fmaf(s.z, k2, -ref)), 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) {
      asm volatile("" : "+v"(buf[k]));
      float f[E::kPerVec];
      E::unpack(buf[k], f);
#pragma unroll
      for (int e = 0; e < E::kPerVec; ++e) f[e] = fast_exp2(fmaf(f[e], k2, -ref));
      acc[k & 3] += tree_sum(f);
    }
    return make_float2(ref, wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3])));
  }
}

// One 16 KiB chunk: (ref, sum 2^(z k - ref)) at T > 0, (max, first index of max) at T = 0.
template <class E, bool kGreedy, bool kVec>
__device__ __forceinline__ float2 chunk_record(const char* rp, int32_t c0, int32_t n, float k2, int lane) {
  u32x4 buf[kVecPerLane];
  if constexpr (kVec) {
    load_chunk<E>(rp, c0, n, lane, buf);
    return record_of<E, kGreedy>(buf, c0, k2, lane);
  } else {
    const SplitEdge s = load_split_chunk<E>(rp, c0, n, lane, buf);
    return record_of_split<E, kGreedy>(buf, s, c0, k2, lane);
  }
}

// The record of a loaded bf16 chunk at T > 0, and the counts of the kHistKeys keys at and below its
// maximum's: out[j / 2] holds the counts of keys kmax - j (low half) and kmax - j - 1 (high half),
// top = kmax.  Only a positive maximum whose window stays above +0 is counted; other chunks (a
// maximum <= 0 or within kHistKeys steps of +0) carry top | kNoCounts and zero counts.  h: the
// wave's kHistKeys counters and kWave spare counters in shared memory.
__device__ __forceinline__ float2 record_counting(u32x4 (&buf)[kVecPerLane], float k2, int lane, uint32_t* h,
                                                  uint32_t* out, uint32_t* top) {
  const float m = chunk_max<Bf16>(buf);
  const uint32_t hm = (uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(m)) >> 16;
  const uint32_t kmax = key16_of_bits(hm);
  const bool counts = hm >= (uint32_t)kHistKeys && hm < 0x8000u;
  if (lane == 0) *top = counts ? kmax : (kmax | kNoCounts);
  if (m == -INFINITY) return make_float2(-INFINITY, 0.0f);
  const float ref = m * k2;
  h[2 * lane] = 0u;
  h[2 * lane + 1] = 0u;
  __builtin_amdgcn_wave_barrier();  // a wave's shared-memory operations complete in order
  const float s = exp_sum<Bf16, true>(buf, k2, ref, counts ? hm : kCountNothing, kHistKeys + lane, h);
  __builtin_amdgcn_wave_barrier();
  out[lane] = h[2 * lane] | (h[2 * lane + 1] << 16);  // a chunk holds at most 8192 logits
  return make_float2(ref, s);
}

// record_counting over a bf16 chunk split at 16-byte boundaries (load_split_chunk): the lane's edge
// element is counted and summed beside the vectors (a lane without one counts the -inf pattern,
// which lands on its spare counter).
__device__ __forceinline__ float2 record_counting_split(u32x4 (&buf)[kVecPerLane], const SplitEdge& se, float k2,
                                                        int lane, uint32_t* h, uint32_t* out, uint32_t* top) {
  float ml = se.z;
#pragma unroll
  for (int k = 0; k < kVecPerLane; ++k) {
    float f[Bf16::kPerVec];
    Bf16::unpack(buf[k], f);
#pragma unroll
    for (int e = 0; e < Bf16::kPerVec; ++e) ml = fmaxf(ml, f[e]);
  }
  const float m = wave_max(ml);
  const uint32_t hm = (uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(m)) >> 16;
  const uint32_t kmax = key16_of_bits(hm);
  const bool counts = hm >= (uint32_t)kHistKeys && hm < 0x8000u;
  if (lane == 0) *top = counts ? kmax : (kmax | kNoCounts);
  if (m == -INFINITY) return make_float2(-INFINITY, 0.0f);
  const float ref = m * k2;
  h[2 * lane] = 0u;
  h[2 * lane + 1] = 0u;
  __builtin_amdgcn_wave_barrier();  // a wave's shared-memory operations complete in order
  const uint32_t hc = counts ? hm : kCountNothing, spare = kHistKeys + lane;
  float s = exp_sum<Bf16, true>(buf, k2, ref, hc, spare, h);
  const uint32_t d = hc - (se.ok ? __float_as_uint(se.z) >> 16 : 0xff80u);
  atomicAdd(&h[d < spare ? d : spare], 1u);
  s += wave_sum(fast_exp2(fmaf(se.z, k2, -ref)));
  __builtin_amdgcn_wave_barrier();
  out[lane] = h[2 * lane] | (h[2 * lane + 1] << 16);
  return make_float2(ref, s);
}

// Residual weight max(p - q, 0) of token v, both sides scaled by the same factor 2^(l2_t - ref_t).
// The draft side is 2^(z_d k - e); e is split into its fp32 rounding e_hi and a remainder that
// enters as the factor q_scale = 2^(e_hi - e), applied by the final fused multiply-add.  A token a
// row does not keep has zero probability on that side: its logit enters as -inf (selecting the
// input rather than the output keeps the masked loops within the register file).
template <class M>
__device__ __forceinline__ float resid_weight(const M& m, float zt, float zd, int32_t v, float k2, float ref_t,
                                              float e_hi, float q_scale) {
  const float p = fast_exp2(fmaf(m.t(zt, v) ? zt : -INFINITY, k2, -ref_t));
  const float q = fast_exp2(fmaf(m.d(zd, v) ? zd : -INFINITY, k2, -e_hi));
  return fmaxf(fmaf(-q, q_scale, p), 0.0f);
}

// Weight of token v in a draw from p itself (the frame 2^(z k - ref_t)).
template <class M>
__device__ __forceinline__ float p_weight(const M& m, float zt, int32_t v, float k2, float ref_t) {
  return fast_exp2(fmaf(m.t(zt, v) ? zt : -INFINITY, k2, -ref_t));
}

// Masses m_c (fp64) of the chunks of one row; returns the chunk holding u * S and the target inside it.
// mass(c) is evaluated by every lane for its chunks; chunks are visited in ascending order.
template <class MassFn>
__device__ __forceinline__ int32_t pick_chunk(int32_t C, double u, MassFn mass, double* target_in_chunk, double* total,
                                              int lane) {
  double S = 0.0;
  for (int32_t c0 = 0; c0 < C; c0 += kWave) S += wave_sum(c0 + lane < C ? mass(c0 + lane) : 0.0);
  *total = S;
  const double U = u * S;
  double carry = 0.0;
  int32_t last_pos = -1;
  double last_before = 0.0;
  for (int32_t c0 = 0; c0 < C; c0 += kWave) {
    const double m = c0 + lane < C ? mass(c0 + lane) : 0.0;
    const double excl = wave_exclusive_scan(m, lane);
    const uint64_t hit = __ballot(c0 + lane < C && carry + excl + m > U);
    if (hit) {
      const int f = __ffsll((unsigned long long)hit) - 1;
      *target_in_chunk = U - (carry + lane_value(excl, f));
      return c0 + f;
    }
    const uint64_t pos = __ballot(c0 + lane < C && m > 0.0);
    if (pos) {
      const int h = 63 - __clzll((long long)pos);
      last_pos = c0 + h;
      last_before = carry + lane_value(excl, h);
    }
    carry += wave_sum(m);
  }
  // rounding left U at or beyond the total: the last chunk with positive mass, targeting its end
  if (last_pos < 0) {
    *target_in_chunk = 0.0;
    return C - 1;
  }
  *target_in_chunk = U - last_before;
  return last_pos;
}

// Residual mass of one chunk of the rejected row pair (16-byte aligned rows): coalesced 16-byte
// loads, fp32 per vector, fp64 across vectors and lanes; each half chunk is summed on its own and the
// halves added, the order of resid_masses_pipelined, so every pass gives a chunk the same mass.
template <class E, class M>
__device__ __forceinline__ double resid_chunk_mass(const M& m, const char* tp, const char* dp, int32_t c0, int32_t n,
                                                   float k2, float ref_t, float e_hi, float q_scale, int lane) {
  const u32x4* tv = reinterpret_cast<const u32x4*>(tp + (int64_t)c0 * E::kBytes);
  const u32x4* dv = reinterpret_cast<const u32x4*>(dp + (int64_t)c0 * E::kBytes);
  const int32_t nvec = n / E::kPerVec;
  constexpr int kHalf = kVecPerLane / 2;  // two halves keep the register footprint at one chunk
  double acc = 0.0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    asm volatile("" ::: "memory");  // keep the second half's loads after the first half's use
    double half = 0.0;
    u32x4 tb[kHalf], db[kHalf];
#pragma unroll
    for (int k = 0; k < kHalf; ++k) {
      const int vi = lane + kWave * (h * kHalf + k);
      tb[k] = load_vec<E>(tv, vi, nvec);
      db[k] = load_vec<E>(dv, vi, nvec);
    }
#pragma unroll
    for (int k = 0; k < kHalf; ++k) {
      float ft[E::kPerVec], fd[E::kPerVec];
      E::unpack(tb[k], ft);
      E::unpack(db[k], fd);
      const int32_t v0 = c0 + (lane + kWave * (h * kHalf + k)) * E::kPerVec;
#pragma unroll
      for (int q = 0; q < E::kPerVec; ++q) ft[q] = resid_weight(m, ft[q], fd[q], v0 + q, k2, ref_t, e_hi, q_scale);
      half += (double)tree_sum(ft);
    }
    acc += half;
  }
  return wave_sum(acc);
}

// How a launch chooses the rule: one greedy or one sampling profile for the batch, or a profile per
// request (the rule of each row then follows its request's temperature).
enum Mode : int { kModeGreedy = 0, kModeSampling = 1, kModeProfiled = 2 };

// The temperature of request i, read through the scalar cache (the index is wave-uniform).
__device__ __forceinline__ float temperature_of(const float* temp_each, int32_t i) {
  return ((const __attribute__((address_space(4))) float*)temp_each)[i];
}

// Waves per row-pass workgroup.  A stream of at least kWideRowUnits chunks (8 workgroups per compute
// unit) runs in workgroups of 8 waves: measured on MI355X, the 256 x 128256 bf16 row pass took 84.2
// against 85.7 us with 4-wave workgroups and the 512 x 151936 greedy pass 118.0 against 119.0 us.
// Smaller grids keep 4 waves, which spread more evenly over the compute units (64 x 32000 bf16:
// 13.4 against 14.6 us with 8), and so do the counting variant, whose per-wave counters 8 waves
// would crowd (91.3 against 93.8 us at top-k 50, top-p 0.9), and the pass with a profile per
// request, which looks up each row's request first (77.5 against 79.1 us).
constexpr int kRowWaves = 4;
constexpr int kWideRowWaves = 8;
constexpr int64_t kWideRowUnits = 16384;

template <class E, int kMode, bool kVec, bool kHist, int kWaves = kRowWaves>
__global__ __launch_bounds__(kWave * kWaves) void row_records(Params P) {
  static_assert(!kHist || (E::kBytes == 2 && kMode != kModeGreedy), "counts: bf16 sampling rows");
  static_assert(kHistKeys == 2 * kWave, "each lane writes one word of two counts");
  __shared__ uint32_t hcnt_all[kHist ? kWaves : 1][kHist ? kHistKeys + kWave : 1];  // counters, then spares
  const int lane = threadIdx.x & (kWave - 1);
  // the unit is wave-uniform; saying so lets the request lookup use scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t u = (int64_t)blockIdx.x * (blockDim.x / kWave) + wave;
  uint32_t* hcnt = hcnt_all[kHist ? wave : 0];
  if (blockIdx.x == 0) {  // once per call: the offsets, and the verdicts' counters from zero
    if (wave == 0) screen_offsets(P, lane);
    for (int32_t j = threadIdx.x; j < P.B; j += blockDim.x) P.split_count[(int64_t)j * kLineWords] = 0u;
  }
  if (u >= P.n_units) return;
  const int32_t slot = (int32_t)(u / P.C);
  const int32_t c = (int32_t)(u - (int64_t)slot * P.C);
  const bool target = slot < P.n_t;
  const char* rp = target ? row_ptr<E>(P.target, slot, P.V) : row_ptr<E>(P.draft, slot - P.n_t, P.V);
  const int32_t c0 = c * E::kChunk;
  const int32_t n = min(E::kChunk, P.V - c0);
  float2 rec;
  if (kHist && u == 0 && lane == 0) P.pending[0] = 0;  // the count kernel appends to an empty list
  if constexpr (kHist && kMode != kModeProfiled) {
    u32x4 buf[kVecPerLane];
    if constexpr (kVec) {
      load_chunk<E>(rp, c0, n, lane, buf);
      rec = record_counting(buf, P.k2, lane, hcnt, P.hist + u * (kHistKeys / 2), P.hist_top + u);
    } else {
      const SplitEdge se = load_split_chunk<E>(rp, c0, n, lane, buf);
      rec = record_counting_split(buf, se, P.k2, lane, hcnt, P.hist + u * (kHistKeys / 2), P.hist_top + u);
    }
  } else if constexpr (kMode != kModeProfiled) {
    rec = chunk_record<E, kMode == kModeGreedy, kVec>(rp, c0, n, P.k2, lane);
  } else {
    // a target row is always read, so its loads go out before the request lookup; a draft row is
    // read only for a request that samples, so the lookup comes first
    const int32_t row = target ? slot : slot - P.n_t;
    if constexpr (kVec) {
      u32x4 buf[kVecPerLane];
      if (target) load_chunk<E>(rp, c0, n, lane, buf);
      const float k2 = k2_of(temperature_of(P.temp_each, request_of_row(P.cu, P.B, row, target)));
      if (!target) {
        if (!(k2 > 0.0f)) return;  // draft row of a greedy or rejected request: never read
        load_chunk<E>(rp, c0, n, lane, buf);
      }
      if constexpr (kHist)
        rec = k2 > 0.0f ? record_counting(buf, k2, lane, hcnt, P.hist + u * (kHistKeys / 2), P.hist_top + u)
                        : record_of<E, true>(buf, c0, 0.0f, lane);
      else
        rec = k2 > 0.0f ? record_of<E, false>(buf, c0, k2, lane) : record_of<E, true>(buf, c0, 0.0f, lane);
    } else {
      const float k2 = k2_of(temperature_of(P.temp_each, request_of_row(P.cu, P.B, row, target)));
      if (!target && !(k2 > 0.0f)) return;
      u32x4 buf[kVecPerLane];
      const SplitEdge se = load_split_chunk<E>(rp, c0, n, lane, buf);
      if constexpr (kHist)
        rec = k2 > 0.0f ? record_counting_split(buf, se, k2, lane, hcnt, P.hist + u * (kHistKeys / 2), P.hist_top + u)
                        : record_of_split<E, true>(buf, se, c0, 0.0f, lane);
      else
        rec = k2 > 0.0f ? record_of_split<E, false>(buf, se, c0, k2, lane)
                        : record_of_split<E, true>(buf, se, c0, 0.0f, lane);
    }
  }
  if (lane == 0) P.part[u] = rec;
}

// Residual chunk masses of a row pair by the waves of one workgroup (16-byte aligned rows).  Wave w
// takes chunks w, w + n_waves, ...; each full chunk is read in two halves, and the loads of the next
// half are issued before the current half is reduced, so every wave keeps one half in flight.  The
// loads of full chunks carry no bounds test (a predicated load would leave the hardware load counter
// uncertain and force a wait for every outstanding load); a row's last, partial chunk goes through
// the bounds-tested path.
template <class E, class M>
__device__ __forceinline__ void resid_masses_pipelined(const M& m, const char* tp, const char* dp, int32_t V, int32_t C,
                                                       float k2, float ref_t, float e_hi, float q_scale,
                                                       double* lds_mass, int lane, int wave, int n_waves) {
  constexpr int kHalf = kVecPerLane / 2;
  struct Half {
    u32x4 t[kHalf], d[kHalf];
  };
  auto load = [&](int32_t c, int h, Half& b) {
    const u32x4* tv = reinterpret_cast<const u32x4*>(tp + (int64_t)c * E::kChunk * E::kBytes);
    const u32x4* dv = reinterpret_cast<const u32x4*>(dp + (int64_t)c * E::kChunk * E::kBytes);
#pragma unroll
    for (int k = 0; k < kHalf; ++k) {
      const int vi = lane + kWave * (h * kHalf + k);
      b.t[k] = tv[vi];
      b.d[k] = dv[vi];
    }
  };
  auto reduce = [&](const Half& b, int32_t c, int h) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kHalf; ++k) {
      float ft[E::kPerVec], fd[E::kPerVec];
      E::unpack(b.t[k], ft);
      E::unpack(b.d[k], fd);
      const int32_t v0 = c * E::kChunk + (lane + kWave * (h * kHalf + k)) * E::kPerVec;
#pragma unroll
      for (int q = 0; q < E::kPerVec; ++q) ft[q] = resid_weight(m, ft[q], fd[q], v0 + q, k2, ref_t, e_hi, q_scale);
      acc += (double)tree_sum(ft);
    }
    return acc;
  };
  const int32_t C_full = V / E::kChunk;  // chunks of kChunk elements
  int32_t c = wave;
  if (c < C_full) {
    Half A, Bh;
    load(c, 0, A);
    asm volatile("" ::: "memory");
    // steady state: every load is unconditional (a load under a branch would leave the load counter
    // unknown at the join and force a wait for every load in flight); the last chunk is peeled off
    for (; c + n_waves < C_full; c += n_waves) {
      load(c, 1, Bh);
      asm volatile("" ::: "memory");  // the second half is in flight while the first is reduced
      double acc = reduce(A, c, 0);
      asm volatile("" : "+v"(acc)::"memory");  // the first half is consumed before its registers reload
      load(c + n_waves, 0, A);
      asm volatile("" ::: "memory");
      acc += reduce(Bh, c, 1);
      asm volatile("" : "+v"(acc)::"memory");
      acc = wave_sum(acc);
      if (lane == 0) lds_mass[c] = acc;
    }
    load(c, 1, Bh);
    asm volatile("" ::: "memory");
    double acc = reduce(A, c, 0);
    asm volatile("" : "+v"(acc)::"memory");
    acc += reduce(Bh, c, 1);
    acc = wave_sum(acc);
    if (lane == 0) lds_mass[c] = acc;
    c += n_waves;
  }
  if (c < C) {  // the partial last chunk, if this wave owns it
    const int32_t c0 = c * E::kChunk;
    const double cm = resid_chunk_mass<E>(m, tp, dp, c0, V - c0, k2, ref_t, e_hi, q_scale, lane);
    if (lane == 0) lds_mass[c] = cm;
  }
}

// Inverse CDF inside kChunks consecutive chunks (16-byte aligned rows) by a whole workgroup: the
// vectors form rows of 64 (vector k*64 + l for lane l), wave w sums rows w, w + n_waves, ..., a scan
// of the row sums picks the row, and the wave that owns it scans its 64 vector sums and walks the
// chosen vector.  Returns the token in the owning wave and -1 in the others.  row_sums holds at least
// 16 kChunks doubles.  kFraction: target is a uniform u in [0, 1), scaled here by the range's total
// weight (the row sums of the first step), which every wave also stores into *total; a residual
// range without positive weight returns -2 in every wave.  With kFraction over a whole row of up to
// four chunks this one pass replaces the mass pass, the pick of a chunk and the search in it.
template <class E, bool kResid, bool kFraction = false, int kChunks = 1, int kWaves = kVerdictWaves, class M>
__device__ __forceinline__ int32_t search_chunk_block(const M& m, const char* trow, const char* drow, int32_t c0,
                                                      int32_t n, double target, float k2, float ref_t, float e_hi,
                                                      float q_scale, double* row_sums, int lane, int wave,
                                                      int n_waves, double* total = nullptr) {
  constexpr int kRows = kVecPerLane * kChunks;  // 16 rows of 64 vectors per chunk
  static_assert(kRows % kWaves == 0 && kRows <= kWave, "whole rows per wave, one scan of the row sums");
  const int32_t nvec = n / E::kPerVec;
  const u32x4* tv = reinterpret_cast<const u32x4*>(trow + (int64_t)c0 * E::kBytes);
  const u32x4* dv = reinterpret_cast<const u32x4*>((kResid ? drow : trow) + (int64_t)c0 * E::kBytes);
  auto weights = [&](const u32x4& t, const u32x4& dd, int32_t v0, float (&w)[E::kPerVec]) {
    float ft[E::kPerVec], fd[E::kPerVec];
    E::unpack(t, ft);
    if constexpr (kResid) E::unpack(dd, fd);
#pragma unroll
    for (int q = 0; q < E::kPerVec; ++q)
      w[q] = kResid ? resid_weight(m, ft[q], fd[q], v0 + q, k2, ref_t, e_hi, q_scale)
                    : p_weight(m, ft[q], v0 + q, k2, ref_t);
  };
  // rows owned by this wave: wave + j n_waves, j < kPer (n_waves == kWaves)
  constexpr int kPer = kRows / kWaves;
  u32x4 t[kPer], dd[kPer];
  float vs[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int vi = (wave + j * n_waves) * kWave + lane;
    t[j] = wave + j * n_waves < kRows ? load_vec<E>(tv, vi, nvec) : neg_inf_vec<E>();
    dd[j] = (kResid && wave + j * n_waves < kRows) ? load_vec<E>(dv, vi, nvec) : neg_inf_vec<E>();
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    float w[E::kPerVec];
    weights(t[j], dd[j], c0 + ((wave + j * n_waves) * kWave + lane) * E::kPerVec, w);
    vs[j] = tree_sum(w);
    const double rs = wave_sum((double)vs[j]);
    if (lane == 0 && wave + j * n_waves < kRows) row_sums[wave + j * n_waves] = rs;
  }
  __syncthreads();
  // every wave scans the 16 row sums the same way
  const double rsum = lane < kRows ? row_sums[lane] : 0.0;
  const double rex = wave_exclusive_scan(rsum, lane);
  double tgt = target;
  if constexpr (kFraction) {
    const double sum = lane_value(rex + rsum, kRows - 1);
    *total = sum;
    if constexpr (kResid) {
      if (!(sum > 0.0)) return -2;
    }
    tgt = target * sum;
  }
  const uint64_t rhit = __ballot(lane < kRows && rex + rsum > tgt);
  const uint64_t rpos = __ballot(lane < kRows && rsum > 0.0);
  if (!rhit && !rpos) return wave == 0 ? c0 + n - 1 : -1;
  const int kr = rhit ? __ffsll((unsigned long long)rhit) - 1 : 63 - __clzll((long long)rpos);
  const int owner = kr % n_waves;
  if (wave != owner) return -1;
  const int j = kr / n_waves;
  const double rest = tgt - lane_value(rex, kr);
  // the owning wave: scan its 64 vector sums of row kr, then walk the chosen vector
  float v = vs[0];  // j is uniform: selects, not an indexed register array
#pragma unroll
  for (int jj = 1; jj < kPer; ++jj)
    if (jj == j) v = vs[jj];
  const double vex = wave_exclusive_scan((double)v, lane);
  const uint64_t vhit = __ballot(rhit && vex + (double)v > rest);
  const uint64_t vpos = __ballot(v > 0.0f);
  const int l = vhit ? __ffsll((unsigned long long)vhit) - 1 : (vpos ? 63 - __clzll((long long)vpos) : 63);
  const int32_t base = c0 + (kr * kWave + lane) * E::kPerVec;
  float w[E::kPerVec];
#pragma unroll
  for (int jj = 0; jj < kPer; ++jj)
    if (jj == j) weights(t[jj], dd[jj], base, w);
  int32_t yl = base + E::kPerVec - 1;
  int32_t last_pos = -1;
  double upto = vex;
  bool found = false;
#pragma unroll
  for (int q = 0; q < E::kPerVec; ++q) {
    upto += (double)w[q];
    if (w[q] > 0.0f) last_pos = base + q;
    if (!found && upto > rest) {
      yl = base + q;
      found = true;
    }
  }
  if (!vhit) yl = last_pos >= 0 ? last_pos : yl;
  return lane_value(yl, l);
}

// ---------------------------------------------------------------------------- rows off the 16-byte grid
// A plan's address as an offset from the row pointer it came from, so that the compiler still
// knows the loads through it read global memory (cast from an integer it would be a flat address:
// flat loads, which also count against the shared-memory wait counter).
__device__ __forceinline__ const char* at_address(const char* base, uintptr_t a) {
  return base + (intptr_t)(a - (uintptr_t)base);
}

// A chunk [c0, c0 + n) of a row pair whose rows are only element-aligned, split on the target row's
// 16-byte grid: `body` vectors from element c0 + head on are aligned in the target row, and the
// draft bytes under vector j are the 16 bytes `shift` past the aligned draft vector dv[j] (one shift
// for the whole pair: the difference of the two rows' addresses modulo 16).  The head and tail
// elements go one per lane.  A vector whose aligned draft pieces would reach outside the draft row
// joins the head or the tail, so every load stays inside its row: at most 2 kPerVec - 1 elements
// on each side, 30 lanes for bf16.  With the target row as its own draft (dp = tp) the split is the
// row pass's.
struct PairSplit {
  int32_t head, body;  // elements before the first vector; vectors
  uint32_t shift;      // bytes from an aligned draft vector to the draft bytes under a target vector
  const u32x4* tv;     // target vector j
  const u32x4* dv;     // draft pieces of vector j: dv[j] and (shift > 0) dv[j + 1]
};
template <class E>
__device__ __forceinline__ PairSplit pair_split(const char* tp, const char* dp, int32_t V, int32_t c0, int32_t n) {
  const split::Plan p = split::pair((uintptr_t)tp, (uintptr_t)dp, E::kBytes, V, c0, n);
  return PairSplit{p.head, p.body, p.shift, reinterpret_cast<const u32x4*>(at_address(tp, p.first)),
                   reinterpret_cast<const u32x4*>(at_address(dp, p.pieces))};
}

// The 16 bytes `shift` bytes into (lo, hi); shift is a multiple of 2 and the same in every lane, so
// the word selects are scalar-conditioned moves and the 2-byte step one v_alignbit per word.  The
// words stay named values: selecting between elements of an array here becomes a select of
// addresses, which puts the array in scratch memory.
__device__ __forceinline__ u32x4 funnel16(const u32x4 lo, const u32x4 hi, uint32_t shift) {
  const bool two = (shift & 8) != 0, one = (shift & 4) != 0;
  const uint32_t bits = (shift & 3) * 8;
  const uint32_t a0 = two ? lo.z : lo.x, a1 = two ? lo.w : lo.y, a2 = two ? hi.x : lo.z, a3 = two ? hi.y : lo.w,
                 a4 = two ? hi.z : hi.x, a5 = two ? hi.w : hi.y;
  const uint32_t c0 = one ? a1 : a0, c1 = one ? a2 : a1, c2 = one ? a3 : a2, c3 = one ? a4 : a3, c4 = one ? a5 : a4;
  return u32x4{__builtin_amdgcn_alignbit(c1, c0, bits), __builtin_amdgcn_alignbit(c2, c1, bits),
               __builtin_amdgcn_alignbit(c3, c2, bits), __builtin_amdgcn_alignbit(c4, c3, bits)};
}

// Body vector j of a split pair (body >= 1): the target vector, -inf from j = body on, and the draft
// bytes under it.  Indices are clamped into the body so that every load is unconditional.
template <class E, bool kResid>
__device__ __forceinline__ void load_split_pair(const PairSplit& s, int j, u32x4& t, u32x4& d) {
  const int jc = min(j, s.body - 1);
  t = s.tv[jc];
  if constexpr (kResid) {
    const u32x4 lo = s.dv[jc];
    const u32x4 hi = s.dv[s.shift != 0 ? jc + 1 : jc];
    d = funnel16(lo, hi, s.shift);
  }
  if (j >= s.body) t = neg_inf_vec<E>();
}

// The chunk-relative element a lane takes at a split's edges (lanes [0, head): the head, then the
// tail), or -1.
template <class Split>
__device__ __forceinline__ int32_t split_edge(const Split& s, int32_t n, int per_vec, int lane) {
  return split::edge(s.head, s.body * per_vec, n, lane);
}

// Residual mass of one chunk of a rejected row pair, by one wave.  The edge elements load first;
// the body goes in quarters of 4 vectors per lane, the loads of the next quarter issued before the
// current one is reduced.  Every quarter loads (indices clamped into the body), so no load sits
// under a branch and the waits count only the loads ahead of the data used.  kVec: 16-byte aligned
// rows (no edges, no shift: one draft vector under each target vector); this form needs fewer
// registers than resid_masses_pipelined and serves the 16-wave verdict workgroups.
template <class E, bool kVec, class M>
__device__ __forceinline__ double resid_chunk_mass_split(const M& m, const char* tp, const char* dp, int32_t V,
                                                         int32_t c0, int32_t n, float k2, float ref_t, float e_hi,
                                                         float q_scale, int lane) {
  const PairSplit s = pair_split<E>(tp, dp, V, c0, n);
  const int32_t e = split_edge(s, n, E::kPerVec, lane);
  float zt = -INFINITY, zd = -INFINITY;
  if (e >= 0) {
    zt = E::at(tp, c0 + e);
    zd = E::at(dp, c0 + e);
  }
  double acc = 0.0;
  if (s.body > 0) {
    constexpr int kParts = 4, kPart = kVecPerLane / kParts;
    struct Stage {
      u32x4 t[kPart], lo[kPart], hi[kPart];
    };
    auto load = [&](int h, Stage& st) {
#pragma unroll
      for (int k = 0; k < kPart; ++k) {
        const int jc = min(lane + kWave * (h * kPart + k), s.body - 1);
        st.t[k] = s.tv[jc];
        st.lo[k] = s.dv[jc];
        if constexpr (!kVec) st.hi[k] = s.dv[s.shift != 0 ? jc + 1 : jc];
      }
    };
    auto pin = [&](Stage& st) {  // the reduction of this stage stays below the loads just issued
#pragma unroll
      for (int k = 0; k < kPart; ++k) {
        if constexpr (kVec) asm volatile("" : "+v"(st.t[k]), "+v"(st.lo[k])::"memory");
        else asm volatile("" : "+v"(st.t[k]), "+v"(st.lo[k]), "+v"(st.hi[k])::"memory");
      }
    };
    auto reduce = [&](const Stage& st, int h) {
      double part = 0.0;
#pragma unroll
      for (int k = 0; k < kPart; ++k) {
        const int j = lane + kWave * (h * kPart + k);
        float ft[E::kPerVec], fd[E::kPerVec];
        E::unpack(j < s.body ? st.t[k] : neg_inf_vec<E>(), ft);
        E::unpack(kVec ? st.lo[k] : funnel16(st.lo[k], st.hi[k], s.shift), fd);
        const int32_t v0 = c0 + s.head + j * E::kPerVec;
#pragma unroll
        for (int q = 0; q < E::kPerVec; ++q) ft[q] = resid_weight(m, ft[q], fd[q], v0 + q, k2, ref_t, e_hi, q_scale);
        part += (double)tree_sum(ft);
      }
      return part;
    };
    Stage A, B;
    load(0, A);
    load(1, B);
    pin(A);
    acc += reduce(A, 0);
    load(2, A);
    pin(B);
    acc += reduce(B, 1);
    load(3, B);
    pin(A);
    acc += reduce(A, 2);
    pin(B);
    acc += reduce(B, 3);
  }
  if (e >= 0) acc += (double)resid_weight(m, zt, zd, c0 + e, k2, ref_t, e_hi, q_scale);
  return wave_sum(acc);
}

// Inverse CDF inside one chunk off the 16-byte grid by a whole workgroup, as search_chunk_block
// with two more segments: the head's elements before the 16 rows of body vectors and the tail's
// after them (wave 0 weighs both).  The scan runs over the 18 segment sums; an edge segment is
// walked by wave 0 lane by lane.  Returns the token in the wave that resolves it, -1 in the
// others.  row_sums holds at least 18 doubles.
template <class E, bool kResid, int kWaves = kVerdictWaves, class M>
__device__ __forceinline__ int32_t search_chunk_split(const M& m, const char* trow, const char* drow, int32_t V,
                                                      int32_t c0, int32_t n, double target, float k2, float ref_t,
                                                      float e_hi, float q_scale, double* row_sums, int lane, int wave,
                                                      int n_waves) {
  constexpr int kRows = kVecPerLane;  // 16 rows of 64 vectors
  constexpr int kPer = kRows / kWaves;
  constexpr int kSeg = kRows + 2;  // the head, the rows, the tail
  const PairSplit s = pair_split<E>(trow, kResid ? drow : trow, V, c0, n);
  auto weights = [&](const u32x4& t, const u32x4& dd, int32_t v0, float (&w)[E::kPerVec]) {
    float ft[E::kPerVec], fd[E::kPerVec];
    E::unpack(t, ft);
    if constexpr (kResid) E::unpack(dd, fd);
#pragma unroll
    for (int q = 0; q < E::kPerVec; ++q)
      w[q] = kResid ? resid_weight(m, ft[q], fd[q], v0 + q, k2, ref_t, e_hi, q_scale)
                    : p_weight(m, ft[q], v0 + q, k2, ref_t);
  };
  const int32_t b0 = c0 + s.head;  // the first body element
  u32x4 t[kPer], dd[kPer];
  float vs[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    t[j] = neg_inf_vec<E>();
    dd[j] = neg_inf_vec<E>();
    if (s.body > 0) load_split_pair<E, kResid>(s, (wave + j * n_waves) * kWave + lane, t[j], dd[j]);
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    float w[E::kPerVec];
    weights(t[j], dd[j], b0 + ((wave + j * n_waves) * kWave + lane) * E::kPerVec, w);
    vs[j] = tree_sum(w);
    const double rs = wave_sum((double)vs[j]);
    if (lane == 0) row_sums[1 + wave + j * n_waves] = rs;
  }
  const int32_t e = split_edge(s, n, E::kPerVec, lane);
  float ew = 0.0f;
  if (wave == 0) {
    if (e >= 0)
      ew = kResid ? resid_weight(m, E::at(trow, c0 + e), E::at(drow, c0 + e), c0 + e, k2, ref_t, e_hi, q_scale)
                  : p_weight(m, E::at(trow, c0 + e), c0 + e, k2, ref_t);
    const double hs = wave_sum(lane < s.head ? (double)ew : 0.0);
    const double ts = wave_sum(lane < s.head ? 0.0 : (double)ew);
    if (lane == 0) {
      row_sums[0] = hs;
      row_sums[kSeg - 1] = ts;
    }
  }
  __syncthreads();
  const double rsum = lane < kSeg ? row_sums[lane] : 0.0;
  const double rex = wave_exclusive_scan(rsum, lane);
  const uint64_t rhit = __ballot(lane < kSeg && rex + rsum > target);
  const uint64_t rpos = __ballot(lane < kSeg && rsum > 0.0);
  if (!rhit && !rpos) return wave == 0 ? c0 + n - 1 : -1;
  const int kr = rhit ? __ffsll((unsigned long long)rhit) - 1 : 63 - __clzll((long long)rpos);
  const double rest = target - lane_value(rex, kr);
  if (kr == 0 || kr == kSeg - 1) {  // an edge segment (positive sum): wave 0 walks its lanes in order
    if (wave != 0) return -1;
    const bool mine = e >= 0 && (kr == 0) == (lane < s.head);
    const double w = mine ? (double)ew : 0.0;
    const double ex = wave_exclusive_scan(w, lane);
    const uint64_t hit = __ballot(rhit && mine && ex + w > rest);
    const uint64_t pos = __ballot(mine && w > 0.0);
    const int l = hit ? __ffsll((unsigned long long)hit) - 1 : 63 - __clzll((long long)pos);
    return lane_value(c0 + e, l);
  }
  const int row = kr - 1;
  const int owner = row % n_waves;
  if (wave != owner) return -1;
  const int j = row / n_waves;
  float v = vs[0];  // j is uniform: selects, not an indexed register array
#pragma unroll
  for (int jj = 1; jj < kPer; ++jj)
    if (jj == j) v = vs[jj];
  const double vex = wave_exclusive_scan((double)v, lane);
  const uint64_t vhit = __ballot(rhit && vex + (double)v > rest);
  const uint64_t vpos = __ballot(v > 0.0f);
  const int l = vhit ? __ffsll((unsigned long long)vhit) - 1 : (vpos ? 63 - __clzll((long long)vpos) : 63);
  const int32_t base = b0 + (row * kWave + lane) * E::kPerVec;
  float w[E::kPerVec];
#pragma unroll
  for (int jj = 0; jj < kPer; ++jj)
    if (jj == j) weights(t[jj], dd[jj], base, w);
  int32_t yl = base + E::kPerVec - 1;
  int32_t last_pos = -1;
  double upto = vex;
  bool found = false;
#pragma unroll
  for (int q = 0; q < E::kPerVec; ++q) {
    upto += (double)w[q];
    if (w[q] > 0.0f) last_pos = base + q;
    if (!found && upto > rest) {
      yl = base + q;
      found = true;
    }
  }
  if (!vhit) yl = last_pos >= 0 ? last_pos : yl;
  return lane_value(yl, l);
}

// ============================================================================ probability-row drafts
// The draft side given as the distributions themselves (SDCP's q_rows: V binary32 values per
// proposed position).  Weights live in the frame 2^(z_t k - ref_t) of the target row; q enters it
// through q_scale = 2^(l2_t - ref_t).

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class M>
__device__ __forceinline__ float resid_weight_q(const M& m, float zt, float qv, int32_t v, float k2, float ref_t,
                                                float q_scale) {
  const float p = fast_exp2(fmaf(m.t(zt, v) ? zt : -INFINITY, k2, -ref_t));
  return fmaxf(fmaf(-qv, q_scale, p), 0.0f);
}

// Four target elements under one 16-byte q vector: 8 bytes of bf16 or 16 bytes of fp32, so that
// target and q loads are both contiguous across the lanes of a wave.
template <class E>
struct Quad;
template <>
struct Quad<Bf16> {
  typedef uint32_t T __attribute__((ext_vector_type(2)));
  __device__ static __forceinline__ void unpack(const T v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};
template <>
struct Quad<F32> {
  typedef u32x4 T;
  __device__ static __forceinline__ void unpack(const T v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};

// Inverse CDF inside one chunk of a (target row, q row) pair by a whole workgroup (16-byte aligned
// rows), laid out as the logit version: rows of 64 vectors, wave w sums rows w and w + n_waves, a
// scan of the row sums picks the row, the owning wave scans its vector sums and walks the vector.
// Returns the token in the owning wave and -1 in the others.  row_sums holds at least 16 doubles.
template <class E, int kWaves = kVerdictWaves, class M>
__device__ __forceinline__ int32_t search_chunk_q_block(const M& m, const char* trow, const float* qrow, int32_t c0,
                                                        int32_t n, double target, float k2, float ref_t,
                                                        float q_scale, double* row_sums, int lane, int wave,
                                                        int n_waves) {
  constexpr int kRows = kVecPerLane;
  constexpr int kQV = E::kPerVec / 4;
  const int32_t nvec = n / E::kPerVec;
  const u32x4* tv = reinterpret_cast<const u32x4*>(trow + (int64_t)c0 * E::kBytes);
  const f32x4* qv = reinterpret_cast<const f32x4*>(qrow + c0);
  auto weights = [&](const u32x4& t, const f32x4 (&q)[kQV], int32_t v0, float (&w)[E::kPerVec]) {
    float ft[E::kPerVec];
    E::unpack(t, ft);
#pragma unroll
    for (int g = 0; g < kQV; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[4 * g + e] = resid_weight_q(m, ft[4 * g + e], q[g][e], v0 + 4 * g + e, k2, ref_t, q_scale);
  };
  constexpr int kPer = kRows / kWaves;  // rows of 64 vectors per wave
  u32x4 t[kPer];
  f32x4 q[kPer][kQV];
  float vs[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int row = wave + j * n_waves;
    const int vi = row * kWave + lane;
    const bool in = row < kRows && vi < nvec;
    t[j] = in ? tv[vi] : neg_inf_vec<E>();
#pragma unroll
    for (int g = 0; g < kQV; ++g) q[j][g] = in ? qv[vi * kQV + g] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    float w[E::kPerVec];
    weights(t[j], q[j], c0 + ((wave + j * n_waves) * kWave + lane) * E::kPerVec, w);
    vs[j] = tree_sum(w);
    const double rs = wave_sum((double)vs[j]);
    if (lane == 0 && wave + j * n_waves < kRows) row_sums[wave + j * n_waves] = rs;
  }
  __syncthreads();
  const double rsum = lane < kRows ? row_sums[lane] : 0.0;
  const double rex = wave_exclusive_scan(rsum, lane);
  const uint64_t rhit = __ballot(lane < kRows && rex + rsum > target);
  const uint64_t rpos = __ballot(lane < kRows && rsum > 0.0);
  if (!rhit && !rpos) return wave == 0 ? c0 + n - 1 : -1;
  const int kr = rhit ? __ffsll((unsigned long long)rhit) - 1 : 63 - __clzll((long long)rpos);
  const int owner = kr % n_waves;
  if (wave != owner) return -1;
  const int j = kr / n_waves;
  const double rest = target - lane_value(rex, kr);
  float v = vs[0];
#pragma unroll
  for (int jj = 1; jj < kPer; ++jj)
    if (jj == j) v = vs[jj];
  const double vex = wave_exclusive_scan((double)v, lane);
  const uint64_t vhit = __ballot(rhit && vex + (double)v > rest);
  const uint64_t vpos = __ballot(v > 0.0f);
  const int l = vhit ? __ffsll((unsigned long long)vhit) - 1 : (vpos ? 63 - __clzll((long long)vpos) : 63);
  const int32_t base = c0 + (kr * kWave + lane) * E::kPerVec;
  float w[E::kPerVec];
#pragma unroll
  for (int jj = 0; jj < kPer; ++jj)
    if (jj == j) weights(t[jj], q[jj], base, w);
  int32_t yl = base + E::kPerVec - 1;
  int32_t last_pos = -1;
  double upto = vex;
  bool found = false;
#pragma unroll
  for (int e = 0; e < E::kPerVec; ++e) {
    upto += (double)w[e];
    if (w[e] > 0.0f) last_pos = base + e;
    if (!found && upto > rest) {
      yl = base + e;
      found = true;
    }
  }
  if (!vhit) yl = last_pos >= 0 ? last_pos : yl;
  return lane_value(yl, l);
}

// ---------------------------------------------------------------------------- q rows off the grid
// A chunk [c0, c0 + n) of a (target row, q row) pair that is not on the 16-byte grid, split on the
// q row's grid: q vector j (4 binary32 values) is aligned, and the 4 target logits under it (8
// bytes of bf16, 16 of fp32) are cut from two aligned pieces of that size by one shift, the same
// for the whole pair.  A quad whose target pieces would reach outside the target row joins the
// head or the tail elements, which go one per lane (at most 7 on each side), so every load stays
// inside its row.
template <class E>
struct QSplit {
  typedef typename Quad<E>::T TQ;
  int32_t head, body;  // elements before the first quad; quads
  uint32_t shift;      // bytes from an aligned target piece to the logits under a quad
  const f32x4* qv;     // q vector j
  const TQ* tv;        // target pieces of quad j: tv[j] and (shift > 0) tv[j + 1]
};
template <class E>
__device__ __forceinline__ QSplit<E> q_split(const char* tp, const float* qp, int32_t V, int32_t c0, int32_t n) {
  const split::Plan p = split::q((uintptr_t)tp, (uintptr_t)qp, E::kBytes, V, c0, n);
  return QSplit<E>{p.head, p.body, p.shift, reinterpret_cast<const f32x4*>(qp + c0 + p.head),
                   reinterpret_cast<const typename Quad<E>::T*>(at_address(tp, p.pieces))};
}

// The 4 target logits `shift` bytes into (lo, hi): 8-byte pieces of bf16 (shift 0, 2, 4 or 6) or
// 16-byte pieces of fp32 (funnel16).
__device__ __forceinline__ Quad<Bf16>::T funnel_quad(const Quad<Bf16>::T lo, const Quad<Bf16>::T hi, uint32_t shift) {
  const bool one = (shift & 4) != 0;
  const uint32_t bits = (shift & 3) * 8;
  const uint32_t c0 = one ? lo.y : lo.x, c1 = one ? hi.x : lo.y, c2 = one ? hi.y : hi.x;
  return Quad<Bf16>::T{__builtin_amdgcn_alignbit(c1, c0, bits), __builtin_amdgcn_alignbit(c2, c1, bits)};
}
__device__ __forceinline__ u32x4 funnel_quad(const u32x4 lo, const u32x4 hi, uint32_t shift) {
  return funnel16(lo, hi, shift);
}
template <class E>
__device__ __forceinline__ typename Quad<E>::T neg_inf_quad() {
  typename Quad<E>::T t;
#pragma unroll
  for (int w = 0; w < (int)(sizeof(t) / 4); ++w) t[w] = E::kNegInfWord;
  return t;
}

// Quad j of a split q pair (body >= 1): the target logits (-inf from j = body on, so the weight
// is 0) and the q vector; indices are clamped into the body so that every load is unconditional.
template <class E>
__device__ __forceinline__ void load_q_quad(const QSplit<E>& s, int j, typename Quad<E>::T& t, f32x4& q) {
  const int jc = min(j, s.body - 1);
  q = s.qv[jc];
  const typename Quad<E>::T lo = s.tv[jc];
  const typename Quad<E>::T hi = s.tv[s.shift != 0 ? jc + 1 : jc];
  t = funnel_quad(lo, hi, s.shift);
  if (j >= s.body) t = neg_inf_quad<E>();
}

// Residual mass of one chunk of a (target row, q row) pair, by one wave: the edge elements load
// first, then the quads in stages of 4 per lane, the loads of the next stage issued before the
// current one is reduced.  kVec: 16-byte aligned rows (no edges, no shift: one target piece per quad).
template <class E, bool kVec, class M>
__device__ __forceinline__ double resid_chunk_mass_q_split(const M& m, const char* tp, const float* qp, int32_t V,
                                                           int32_t c0, int32_t n, float k2, float ref_t, float q_scale,
                                                           int lane) {
  typedef typename Quad<E>::T TQ;
  const QSplit<E> s = q_split<E>(tp, qp, V, c0, n);
  const int32_t e = split_edge(s, n, 4, lane);
  float zt = -INFINITY, qe = 0.0f;
  if (e >= 0) {
    zt = E::at(tp, c0 + e);
    qe = qp[c0 + e];
  }
  double acc = 0.0;
  if (s.body > 0) {
    constexpr int kQuadsPerLane = E::kChunk / 4 / kWave;  // 32 (bf16) or 16 (fp32)
    constexpr int kPart = 4, kParts = kQuadsPerLane / kPart;
    struct Stage {
      TQ lo[kPart], hi[kPart];
      f32x4 q[kPart];
    };
    auto load = [&](int h, Stage& st) {
#pragma unroll
      for (int k = 0; k < kPart; ++k) {
        const int jc = min(lane + kWave * (h * kPart + k), s.body - 1);
        st.q[k] = s.qv[jc];
        st.lo[k] = s.tv[jc];
        if constexpr (!kVec) st.hi[k] = s.tv[s.shift != 0 ? jc + 1 : jc];
      }
    };
    auto pin = [&](Stage& st) {  // the reduction of this stage stays below the loads just issued
#pragma unroll
      for (int k = 0; k < kPart; ++k) {
        if constexpr (kVec) asm volatile("" : "+v"(st.lo[k]), "+v"(st.q[k])::"memory");
        else asm volatile("" : "+v"(st.lo[k]), "+v"(st.hi[k]), "+v"(st.q[k])::"memory");
      }
    };
    auto reduce = [&](const Stage& st, int h) {  // quad by quad: few weights live at once
      float part = 0.0f;
#pragma unroll
      for (int k = 0; k < kPart; ++k) {
        const int j = lane + kWave * (h * kPart + k);
        float ft[4], w[4];
        const TQ t = kVec ? st.lo[k] : funnel_quad(st.lo[k], st.hi[k], s.shift);
        Quad<E>::unpack(j < s.body ? t : neg_inf_quad<E>(), ft);
        const int32_t v0 = c0 + s.head + 4 * j;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = resid_weight_q(m, ft[q], st.q[k][q], v0 + q, k2, ref_t, q_scale);
        part += tree_sum(w);
      }
      return (double)part;
    };
    Stage A, B;
    load(0, A);
#pragma unroll
    for (int h = 0; h < kParts; h += 2) {
      load(h + 1, B);
      pin(A);
      acc += reduce(A, h);
      if (h + 2 < kParts) load(h + 2, A);
      pin(B);
      acc += reduce(B, h + 1);
    }
  }
  if (e >= 0) acc += (double)resid_weight_q(m, zt, qe, c0 + e, k2, ref_t, q_scale);
  return wave_sum(acc);
}

// Inverse CDF inside one chunk of a (target row, q row) pair off the 16-byte grid by a whole
// workgroup: the quads form rows of 64 (quad r*64 + l for lane l), wave w sums rows w,
// w + n_waves, ..., and the head's and tail's elements are two more segments before and after
// them, weighed and walked by wave 0 as in search_chunk_split.  Returns the token in the wave that
// resolves it, -1 in the others.  row_sums holds at least 34 doubles.
template <class E, int kWaves = kVerdictWaves, class M>
__device__ __forceinline__ int32_t search_chunk_q_split(const M& m, const char* trow, const float* qrow, int32_t V,
                                                        int32_t c0, int32_t n, double target, float k2, float ref_t,
                                                        float q_scale, double* row_sums, int lane, int wave,
                                                        int n_waves) {
  typedef typename Quad<E>::T TQ;
  constexpr int kRows = E::kChunk / 4 / kWave;  // rows of 64 quads: 32 (bf16) or 16 (fp32)
  constexpr int kPer = kRows / kWaves;
  constexpr int kSeg = kRows + 2;  // the head, the rows, the tail
  static_assert(kRows % kWaves == 0 && kSeg <= kWave, "whole rows per wave, one scan of the segments");
  const QSplit<E> s = q_split<E>(trow, qrow, V, c0, n);
  const int32_t b0 = c0 + s.head;
  auto weights = [&](const TQ& t, const f32x4& q, int32_t v0, float (&w)[4]) {
    float ft[4];
    Quad<E>::unpack(t, ft);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = resid_weight_q(m, ft[e], q[e], v0 + e, k2, ref_t, q_scale);
  };
  TQ t[kPer];
  f32x4 q[kPer];
  float vs[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    t[j] = neg_inf_quad<E>();
    q[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (s.body > 0) load_q_quad<E>(s, (wave + j * n_waves) * kWave + lane, t[j], q[j]);
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    float w[4];
    weights(t[j], q[j], b0 + 4 * ((wave + j * n_waves) * kWave + lane), w);
    vs[j] = (w[0] + w[1]) + (w[2] + w[3]);
    const double rs = wave_sum((double)vs[j]);
    if (lane == 0) row_sums[1 + wave + j * n_waves] = rs;
  }
  const int32_t e = split_edge(s, n, 4, lane);
  float ew = 0.0f;
  if (wave == 0) {
    if (e >= 0) ew = resid_weight_q(m, E::at(trow, c0 + e), qrow[c0 + e], c0 + e, k2, ref_t, q_scale);
    const double hs = wave_sum(lane < s.head ? (double)ew : 0.0);
    const double ts = wave_sum(lane < s.head ? 0.0 : (double)ew);
    if (lane == 0) {
      row_sums[0] = hs;
      row_sums[kSeg - 1] = ts;
    }
  }
  __syncthreads();
  const double rsum = lane < kSeg ? row_sums[lane] : 0.0;
  const double rex = wave_exclusive_scan(rsum, lane);
  const uint64_t rhit = __ballot(lane < kSeg && rex + rsum > target);
  const uint64_t rpos = __ballot(lane < kSeg && rsum > 0.0);
  if (!rhit && !rpos) return wave == 0 ? c0 + n - 1 : -1;
  const int kr = rhit ? __ffsll((unsigned long long)rhit) - 1 : 63 - __clzll((long long)rpos);
  const double rest = target - lane_value(rex, kr);
  if (kr == 0 || kr == kSeg - 1) {  // an edge segment (positive sum): wave 0 walks its lanes in order
    if (wave != 0) return -1;
    const bool mine = e >= 0 && (kr == 0) == (lane < s.head);
    const double w = mine ? (double)ew : 0.0;
    const double ex = wave_exclusive_scan(w, lane);
    const uint64_t hit = __ballot(rhit && mine && ex + w > rest);
    const uint64_t pos = __ballot(mine && w > 0.0);
    const int l = hit ? __ffsll((unsigned long long)hit) - 1 : 63 - __clzll((long long)pos);
    return lane_value(c0 + e, l);
  }
  const int row = kr - 1;
  if (wave != row % n_waves) return -1;
  const int j = row / n_waves;
  float v = vs[0];  // j is uniform: selects, not an indexed register array
#pragma unroll
  for (int jj = 1; jj < kPer; ++jj)
    if (jj == j) v = vs[jj];
  const double vex = wave_exclusive_scan((double)v, lane);
  const uint64_t vhit = __ballot(rhit && vex + (double)v > rest);
  const uint64_t vpos = __ballot(v > 0.0f);
  const int l = vhit ? __ffsll((unsigned long long)vhit) - 1 : (vpos ? 63 - __clzll((long long)vpos) : 63);
  const int32_t base = b0 + 4 * (row * kWave + lane);
  float w[4];
#pragma unroll
  for (int jj = 0; jj < kPer; ++jj)
    if (jj == j) weights(t[jj], q[jj], base, w);
  int32_t yl = base + 3;
  int32_t last_pos = -1;
  double upto = vex;
  bool found = false;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    upto += (double)w[e2];
    if (w[e2] > 0.0f) last_pos = base + e2;
    if (!found && upto > rest) {
      yl = base + e2;
      found = true;
    }
  }
  if (!vhit) yl = last_pos >= 0 ? last_pos : yl;
  return lane_value(yl, l);
}

// ============================================================================ 2. truncation
// SDCP ("Speculative Decoding Coordination Protocol (SDCP)", section "Session Contract") defines p
// as the model's distribution after temperature, then top-k, then top-p.  Each logit row gets its
// cut: the value of the last kept rank and how many of its copies are kept (ranks that tie on a
// logit differ only in token id).  Both follow from counts over an order-preserving key of the
// logits: every copy of a key has the same mass, so counts give masses.
//
//  row_cuts_counted  bf16 rows: the row pass has counted, per chunk, the 128 keys
//                    at and below the chunk maximum's (section 1); one wave per row sums them into
//                    the row's top 128 keys and settles the cut when it lands there.  Other rows go
//                    on a list for row_cuts.
//  row_cuts          one workgroup per row (or per listed row): bf16 rows count the 4096 keys below
//                    the row maximum's in one pass and settle cuts that land there; everything else
//                    goes through an exact radix select: per digit level, counts and fixed-point
//                    masses of the logits that share the higher digits, and the level's scan picks
//                    the digit holding the top_k-th rank (top-k) or where the running mass reaches
//                    the nucleus mass (top-p).
//
// Masses are 2^(z k - R) as fixed-point integers (R = fl(max z * k)): integer sums do not depend on
// the order of the atomic adds, so the cut is the same on every run.  The last steps (finish_cut)
// find the token id of the last kept copy and rewrite each chunk record's mass to the mass of the
// chunk's kept tokens, so the verdict kernel's fold yields the truncated normaliser unchanged.

constexpr int kCutWaves = 8;
constexpr int kCutThreads = kWave * kCutWaves;  // several workgroups per CU: rows overlap
constexpr int kRadixBins = 1 << 11;             // the widest digit
constexpr int kBinsPerThread = kRadixBins / kCutThreads;
constexpr int kRegionKeys = 4096;               // bf16 keys counted one by one below the maximum's
constexpr int kKeysPerThread = kRegionKeys / kCutThreads;
constexpr int kTopKeys = 256;   // the window's top keys, also counted per chunk ...
constexpr int kTopChunks = 32;  // ... for rows of up to 32 chunks (32 KiB of LDS)
constexpr float kFixScale = 0x1.0p37f;          // masses <= ~1 as integers: V 2^37 < 2^63

// Digits of the order key, most significant first: bf16 keys carry 16 bits (11 + 5), binary32
// keys 32 (11 + 11 + 10).
template <class E>
struct Radix;
template <>
struct Radix<Bf16> {
  static constexpr int kLevels = 2;
  __device__ static constexpr int shift(int L) { return L == 0 ? 21 : 16; }
  __device__ static constexpr int width(int L) { return L == 0 ? 11 : 5; }
};
template <>
struct Radix<F32> {
  static constexpr int kLevels = 3;
  __device__ static constexpr int shift(int L) { return L == 0 ? 21 : (L == 1 ? 10 : 0); }
  __device__ static constexpr int width(int L) { return L == 2 ? 10 : 11; }
};

// Order-preserving key: a larger logit has a larger key, and -0 shares the key of +0 (they are
// equal logits).  key_logit inverts it.
__device__ __forceinline__ uint32_t order_key(float z) {
  const uint32_t b = z == 0.0f ? 0u : __float_as_uint(z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint64_t fixed_mass(float z, float k2, float R) {
  return (uint64_t)(fast_exp2(fmaf(z, k2, -R)) * kFixScale);
}


struct CutShared {
  uint32_t wave_cnt[kCutWaves];
  uint64_t wave_mass[kCutWaves];
  double wave_real[kCutWaves];
  float wave_ref[kCutWaves];
  int32_t cand, last;
  uint32_t top;
  uint32_t pick_digit, pick_cnt_above, pick_cnt;
  uint64_t pick_mass_above;
};

// Exclusive scan over the workgroup's threads, in thread order, of a (count, mass) pair, and the
// totals.
__device__ __forceinline__ void block_scan(uint32_t c, uint64_t m, uint32_t& c_before, uint64_t& m_before,
                                           uint64_t& c_total, uint64_t& m_total, CutShared& sh) {
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  uint32_t ci = c;
  uint64_t mi = m;
  ci = wave_inclusive_scan(ci);
  mi = wave_inclusive_scan(mi);
  if (lane == kWave - 1) {
    sh.wave_cnt[wave] = ci;
    sh.wave_mass[wave] = mi;
  }
  __syncthreads();
  uint32_t cb = 0u;
  uint64_t mb = 0ull, ct = 0ull, mt = 0ull;
  for (int w = 0; w < kCutWaves; ++w) {
    if (w < wave) {
      cb += sh.wave_cnt[w];
      mb += sh.wave_mass[w];
    }
    ct += sh.wave_cnt[w];
    mt += sh.wave_mass[w];
  }
  __syncthreads();  // the wave totals may be overwritten after this
  c_before = cb + ci - c;
  m_before = mb + mi - m;
  c_total = ct;
  m_total = mt;
}

// A selection's outcome: the key of the last kept logit value, how many tokens rank above that
// value, their mass, and how many tokens carry the value.
struct Selected {
  uint32_t key;
  uint32_t cnt_above;
  uint64_t mass_above;
  uint32_t ties;
};

// The fewest copies (at least one) of a value of per-copy mass e that bring the running mass from
// above to target; the selected value's copies reach it, so the estimate starts within a rounding
// step of the answer and the corrections are short.  Capped at the copies there are.
__device__ __forceinline__ uint32_t copies_to_reach(uint64_t above, uint64_t e, uint32_t ties, double target) {
  uint64_t n = 1ull;
  if (e > 0ull && (double)(above + e) < target) {
    const double est = ceil((target - (double)above) / (double)e);
    n = est >= (double)ties ? (uint64_t)ties : (uint64_t)est;
    while (n > 1ull && (double)(above + (n - 1ull) * e) >= target) --n;
    while (n < ties && (double)(above + n * e) < target) ++n;
  }
  return (uint32_t)(n > ties ? ties : n);
}

// The bin a selection lands in, scanning bins from the largest down: by count, the bin holding
// the need-th logit; by mass, the first non-empty bin where mass_before plus the running mass
// reaches target; failing both (rounding), the last non-empty bin.  bins[p] for p in rank order is
// bin nb - 1 - p; thread t takes ranks kPer t .. kPer t + kPer - 1.  Leaves the bin, the count and
// mass of the bins before it, and its count in sh.pick_*.
template <int kPer, class BinCount, class BinMass>
__device__ __forceinline__ void select_bin(int nb, BinCount count_of, BinMass mass_of, bool by_mass, uint32_t need,
                                           double target, uint64_t mass_before, CutShared& sh) {
  const int t = threadIdx.x;
  if (t == 0) {
    sh.cand = INT32_MAX;
    sh.last = -1;
  }
  uint32_t c[kPer];
  uint64_t m[kPer];
  uint32_t csum = 0u;
  uint64_t msum = 0ull;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int p = kPer * t + q;
    c[q] = p < nb ? count_of(nb - 1 - p) : 0u;
    m[q] = p < nb ? mass_of(nb - 1 - p) : 0ull;
    csum += c[q];
    msum += m[q];
  }
  uint32_t cb;
  uint64_t mb, ct, mt;
  block_scan(csum, msum, cb, mb, ct, mt, sh);
  int cand = INT32_MAX, last = -1;
  uint32_t run_c = cb;
  uint64_t run_m = mb;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int p = kPer * t + q;
    const bool hit = by_mass ? (c[q] > 0u && (double)(mass_before + run_m + m[q]) >= target)
                             : (run_c < need && need <= run_c + c[q]);
    if (p < nb && hit && cand == INT32_MAX) cand = p;
    if (p < nb && c[q] > 0u) last = p;
    run_c += c[q];
    run_m += m[q];
  }
  atomicMin(&sh.cand, cand);
  atomicMax(&sh.last, last);
  __syncthreads();
  const int ps = sh.cand != INT32_MAX ? sh.cand : max(sh.last, 0);
  if (ps / kPer == t) {
    uint32_t above_c = cb;
    uint64_t above_m = mb;
    for (int q = 0; q < ps - kPer * t; ++q) {
      above_c += c[q];
      above_m += m[q];
    }
    sh.pick_digit = (uint32_t)(nb - 1 - ps);
    sh.pick_cnt_above = above_c;
    sh.pick_mass_above = above_m;
    sh.pick_cnt = c[ps - kPer * t];
  }
  __syncthreads();
}

// Every logit of a row, visited by the workgroup (f(z, bits, v); bits are the logit's raw 16 bits
// for bf16 rows).  The row goes by 16-byte vectors, as the row pass reads it: wave w takes chunks w,
// w + 8, ... of the vectors, each loaded whole (16 vectors per lane, 16 KiB in flight per wave)
// before it is visited; the partial last chunk goes through bounds-tested loads.  A row that is
// only element-aligned (kVec false) starts its vectors at its first 16-byte boundary; the elements
// before it and after the last whole vector are visited one per thread.
template <class E, bool kVec, class F>
__device__ __forceinline__ void for_each_logit(const char* rp, int32_t V, F f) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  auto visit = [&](const u32x4& v, int32_t v0) {  // v0: the row index of the vector's first element
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (E::kBytes == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f(__uint_as_float(w[q] << 16), w[q] & 0xffffu, v0 + 2 * q);
        f(__uint_as_float(w[q] & 0xffff0000u), w[q] >> 16, v0 + 2 * q + 1);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) f(__uint_as_float(w[q]), 0u, v0 + q);
    }
  };
  auto visit_one = [&](int32_t v) {
    if constexpr (E::kBytes == 2) {
      const uint32_t h = reinterpret_cast<const uint16_t*>(rp)[v];
      f(__uint_as_float(h << 16), h, v);
    } else {
      f(E::at(rp, v), 0u, v);
    }
  };
  int32_t head = 0;  // elements before the first 16-byte boundary
  if constexpr (!kVec) head = split::to_boundary((uintptr_t)rp, E::kBytes, V);
  const u32x4* vp = reinterpret_cast<const u32x4*>(rp + (int64_t)head * E::kBytes);
  constexpr int32_t kVecPerChunk = E::kChunk / E::kPerVec;
  const int32_t nvec = (V - head) / E::kPerVec, C_full = nvec / kVecPerChunk;
  for (int32_t c = wave; c < C_full; c += kCutWaves) {
    const u32x4* cp = vp + (int64_t)c * kVecPerChunk;
    u32x4 buf[kVecPerLane];
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) buf[k] = cp[lane + kWave * k];
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) {
      // one vector at a time: its keys are not all computed ahead of the atomics
      asm volatile("" : "+v"(buf[k])::"memory");
      visit(buf[k], head + (c * kVecPerChunk + lane + kWave * k) * E::kPerVec);
    }
  }
  if (C_full * kVecPerChunk < nvec && C_full % kCutWaves == wave) {  // the partial last chunk
    for (int32_t vi = C_full * kVecPerChunk + lane; vi < nvec; vi += kWave) visit(vp[vi], head + vi * E::kPerVec);
  }
  if constexpr (!kVec) {  // the head, then the tail after the last whole vector
    const int32_t tail0 = head + nvec * E::kPerVec;
    const int t = threadIdx.x;
    if (t < head) visit_one(t);
    else if (t - head < V - tail0) visit_one(tail0 + (t - head));
  }
}

// bf16 rows: the counts of the keys bottom .. top (cnt[key - bottom], at most kRegionKeys keys) by a
// pass over the row.  With top_cnt (rows of at most kTopChunks chunks) the top kTopKeys keys are also
// counted per chunk: top_cnt[c * kTopKeys + (top - key)].  Returns false when a logit lies above top.
template <bool kVec>
__device__ __forceinline__ bool window_count(const char* rp, int32_t V, int32_t C, uint32_t top, uint32_t bottom,
                                             uint32_t* cnt, uint32_t* top_cnt, CutShared& sh) {
  const int t = threadIdx.x;
  for (int j = t; j < kRegionKeys; j += kCutThreads) cnt[j] = 0u;
  if (top_cnt)
    for (int j = t; j < C * kTopKeys; j += kCutThreads) top_cnt[j] = 0u;
  __syncthreads();
  uint32_t above = 0u;
  for_each_logit<Bf16, kVec>(rp, V, [&](float, uint32_t h, int32_t v) {
    const uint32_t key = key16_of_bits(h);
    if (key > top) {
      ++above;
    } else if (key >= bottom) {
      atomicAdd(&cnt[key - bottom], 1u);
      if (top_cnt && top - key < (uint32_t)kTopKeys)
        atomicAdd(&top_cnt[(v / Bf16::kChunk) * kTopKeys + (top - key)], 1u);
    }
  });
  uint32_t cb;
  uint64_t mb, ct, mt;
  block_scan(above, 0ull, cb, mb, ct, mt, sh);
  return ct == 0ull;
}

// The cut of top-k, then top-p, from the counts of the keys bottom .. top (bf16 rows; every copy of
// a key has the same mass, so counts give masses).  With top-p over the whole row (no top-k) the
// nucleus mass is a share of the row's mass, folded from the chunk records (binary32 chunk sums,
// fp64 across chunks; their relative error stays below 1e-6).  Returns true with the cut in s /
// n_eq when the selection ends on a counted key; false when it lies below them.
__device__ __forceinline__ bool window_pick(const uint32_t* cnt, uint32_t top, uint32_t bottom, int32_t C,
                                            const float2* rec, float k2, float R, bool by_k, int32_t top_k,
                                            bool by_p, int32_t milli, CutShared& sh, Selected& s, uint32_t& n_eq) {
  const int t = threadIdx.x;
  // the row's mass in fixed point, from the chunk records
  double part = 0.0;
  for (int32_t c = t; c < C; c += kCutThreads)
    if (rec[c].y > 0.0f) part += (double)rec[c].y * exp2((double)rec[c].x - (double)R);
  part = wave_sum(part);
  if ((t & (kWave - 1)) == 0) sh.wave_real[t / kWave] = part;
  __syncthreads();
  double row_mass = 0.0;
  for (int w = 0; w < kCutWaves; ++w) row_mass += sh.wave_real[w];
  const uint64_t mass_all = (uint64_t)(row_mass * (double)kFixScale);
  // runs of kKeysPerThread keys, thread order = rank order
  const int32_t hi = (int32_t)top - kKeysPerThread * t;
  uint32_t c = 0u;
  uint64_t m = 0ull;
#pragma unroll
  for (int j = 0; j < kKeysPerThread; ++j) {
    const int32_t key = hi - j;
    const uint32_t n = key >= (int32_t)bottom ? cnt[key - (int32_t)bottom] : 0u;
    c += n;
    if (by_p && n) m += (uint64_t)n * fixed_mass(key_logit(key16_to_key((uint32_t)key)), k2, R);
  }
  uint32_t cb;
  uint64_t mb, ct, mt;
  block_scan(c, m, cb, mb, ct, mt, sh);
  if (by_k && (uint64_t)top_k > ct) return false;  // the top-k cut lies below the window
  // the key inside a run where a selection lands, by the run's owner
  auto pick_in_run = [&](bool by_mass, uint32_t need, double target) {
    uint32_t run_c = cb;
    uint64_t run_m = mb;
    int32_t last = -1;
    for (int j = 0; j < kKeysPerThread; ++j) {
      const int32_t key = hi - j;
      const uint32_t n = key >= (int32_t)bottom ? cnt[key - (int32_t)bottom] : 0u;
      const uint64_t mm = (by_p && n) ? (uint64_t)n * fixed_mass(key_logit(key16_to_key((uint32_t)key)), k2, R) : 0ull;
      const bool hit = by_mass ? (n > 0u && (double)(run_m + mm) >= target) : (run_c < need && need <= run_c + n);
      if (n > 0u) last = j;
      if (hit || (j == kKeysPerThread - 1 && by_mass)) {
        if (!hit) {  // rounding left the target unreached: the last non-empty key of the run
          run_c = cb;
          run_m = mb;
          for (int q = 0; q < last; ++q) {
            const int32_t kq = hi - q;
            const uint32_t nq = kq >= (int32_t)bottom ? cnt[kq - (int32_t)bottom] : 0u;
            run_c += nq;
            if (by_p && nq) run_m += (uint64_t)nq * fixed_mass(key_logit(key16_to_key((uint32_t)kq)), k2, R);
          }
          const int32_t kl = hi - max(last, 0);
          sh.pick_digit = (uint32_t)kl;
          sh.pick_cnt_above = run_c;
          sh.pick_mass_above = run_m;
          sh.pick_cnt = kl >= (int32_t)bottom ? cnt[kl - (int32_t)bottom] : 0u;
          return;
        }
        sh.pick_digit = (uint32_t)key;
        sh.pick_cnt_above = run_c;
        sh.pick_mass_above = run_m;
        sh.pick_cnt = n;
        return;
      }
      run_c += n;
      run_m += mm;
    }
  };
  // top-k: the run holding rank top_k
  uint64_t mass_k = mass_all;
  if (by_k) {
    if (cb < (uint32_t)top_k && (uint32_t)top_k <= cb + c) pick_in_run(false, (uint32_t)top_k, 0.0);
    __syncthreads();
    s = Selected{key16_to_key(sh.pick_digit), sh.pick_cnt_above, sh.pick_mass_above, sh.pick_cnt};
    n_eq = (uint32_t)top_k - s.cnt_above;
    mass_k = s.mass_above + (uint64_t)n_eq * fixed_mass(key_logit(s.key), k2, R);
    __syncthreads();
  }
  if (!by_p) return true;
  // top-p: the first run (in rank order) where the running mass reaches the target
  const double target = (double)mass_k * ((double)milli / 1000.0);
  if (t == 0) sh.cand = INT32_MAX;
  __syncthreads();
  if (c > 0u && (double)(mb + m) >= target) atomicMin(&sh.cand, t);
  __syncthreads();
  const int owner = sh.cand;
  __syncthreads();
  if (owner == INT32_MAX) return false;  // the nucleus reaches below the window
  if (t == owner) pick_in_run(true, 0u, target);
  __syncthreads();
  const Selected sp{key16_to_key(sh.pick_digit), sh.pick_cnt_above, sh.pick_mass_above, sh.pick_cnt};
  __syncthreads();
  uint32_t n = copies_to_reach(sp.mass_above, fixed_mass(key_logit(sp.key), k2, R), sp.ties, target);
  if (by_k && sp.key == s.key && n > n_eq) n = n_eq;
  s = sp;
  n_eq = n;
  return true;
}

// The histogram of one radix digit level over the logits whose higher digits equal prefix: counts,
// and (with_mass) fixed-point masses.
template <class E, bool kVec>
__device__ __forceinline__ void histogram(const char* rp, int32_t V, float k2, float R, int L, uint32_t prefix,
                                          bool with_mass, uint32_t* cnt, uint64_t* mass) {
  const int shift = Radix<E>::shift(L), nb = 1 << Radix<E>::width(L);
  const int hi = shift + Radix<E>::width(L);
  for (int b = threadIdx.x; b < nb; b += kCutThreads) {
    cnt[b] = 0u;
    mass[b] = 0ull;
  }
  __syncthreads();
  for_each_logit<E, kVec>(rp, V, [&](float z, uint32_t, int32_t) {
    const uint32_t key = order_key(z);
    if (L > 0 && (key >> hi) != prefix) return;
    const uint32_t d = (key >> shift) & (uint32_t)(nb - 1);
    atomicAdd(&cnt[d], 1u);
    if (with_mass) atomicAdd(reinterpret_cast<unsigned long long*>(&mass[d]), (unsigned long long)fixed_mass(z, k2, R));
  });
  __syncthreads();
}

// The exact radix select of top-k, then top-p (any row).  cnt0 / mass0 hold level 0 for the whole
// selection, cntL / massL the deeper level last built (reused by top-p when its digits agree).
template <class E, bool kVec>
__device__ __forceinline__ void radix_select(const char* rp, int32_t V, float k2, float R, bool by_k, int32_t top_k,
                                             bool by_p, int32_t milli, unsigned char* smem, CutShared& sh,
                                             Selected& s, uint32_t& n_eq) {
  uint32_t* cnt0 = reinterpret_cast<uint32_t*>(smem);
  uint64_t* mass0 = reinterpret_cast<uint64_t*>(smem + 8 * 1024);
  uint32_t* cntL = reinterpret_cast<uint32_t*>(smem + 24 * 1024);
  uint64_t* massL = reinterpret_cast<uint64_t*>(smem + 32 * 1024);
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  histogram<E, kVec>(rp, V, k2, R, 0, 0u, by_p, cnt0, mass0);
  int held_level = -1;
  uint32_t held_prefix = 0u;
  constexpr int kLast = Radix<E>::kLevels - 1;
  auto run = [&](bool by_mass, uint32_t need, double target_mass) {
    uint32_t prefix = 0u, cnt_above = 0u, ties = 0u;
    uint64_t mass_above = 0ull;
    for (int L = 0; L <= kLast; ++L) {
      const uint32_t* c = cnt0;
      const uint64_t* m = mass0;
      if (L > 0) {
        if (held_level != L || held_prefix != prefix) {
          histogram<E, kVec>(rp, V, k2, R, L, prefix, by_p, cntL, massL);
          held_level = L;
          held_prefix = prefix;
        }
        c = cntL;
        m = massL;
      }
      select_bin<kBinsPerThread>(
          1 << Radix<E>::width(L), [&](int b) { return c[b]; }, [&](int b) { return m[b]; }, by_mass,
          need - cnt_above, target_mass, mass_above, sh);
      cnt_above += sh.pick_cnt_above;
      mass_above += sh.pick_mass_above;
      ties = sh.pick_cnt;
      prefix = (prefix << Radix<E>::width(L)) | sh.pick_digit;
      __syncthreads();
    }
    constexpr int sl = Radix<E>::shift(kLast);
    uint32_t key = prefix;
    if constexpr (sl > 0) key = (prefix << sl) | (((prefix >> (31 - sl)) & 1u) ? 0u : ((1u << sl) - 1u));
    return Selected{key, cnt_above, mass_above, ties};
  };
  uint64_t mass_k = 0ull;
  if (by_k) {
    s = run(false, (uint32_t)top_k, 0.0);
    n_eq = (uint32_t)top_k - s.cnt_above;
    mass_k = s.mass_above + (uint64_t)n_eq * fixed_mass(key_logit(s.key), k2, R);
  } else {
    uint64_t part = 0ull;
    for (int b = t; b < kRadixBins; b += kCutThreads) part += mass0[b];
    part = wave_sum_u64(part);
    if (lane == 0) sh.wave_mass[wave] = part;
    __syncthreads();
    for (int w = 0; w < kCutWaves; ++w) mass_k += sh.wave_mass[w];
    __syncthreads();
  }
  if (by_p) {
    const double target_mass = (double)mass_k * ((double)milli / 1000.0);
    const Selected sp = run(true, 0u, target_mass);
    uint32_t n = copies_to_reach(sp.mass_above, fixed_mass(key_logit(sp.key), k2, R), sp.ties, target_mass);
    if (by_k && sp.key == s.key && n > n_eq) n = n_eq;
    s = sp;
    n_eq = n;
  }
}

// Per chunk of a truncated row: the mass of its tokens above the cut value kappa (2^(z k - ref_c),
// binary32, in the chunk record's frame) and the copies of kappa.  Wave w takes chunks w, w + 8, ...,
// each loaded whole before it is summed; the partial last chunk goes through bounds-tested loads.
template <class E, bool kVec>
__device__ __forceinline__ void chunk_pass(const char* rp, int32_t V, int32_t C, const float2* rec, float kappa,
                                           float k2, float* strict, uint32_t* copies, int lane, int wave) {
  for (int32_t c = wave; c < C; c += kCutWaves) {
    const int32_t c0 = c * E::kChunk, n = min(E::kChunk, V - c0);
    const float ref_c = rec[c].x;
    float acc = 0.0f;
    uint32_t cp = 0u;
    auto take = [&](float z) {
      if (z > kappa) acc += fast_exp2(fmaf(z, k2, -ref_c));
      cp += z == kappa ? 1u : 0u;
    };
    if (kVec && n == E::kChunk) {
      const u32x4* vp = reinterpret_cast<const u32x4*>(rp + (int64_t)c0 * E::kBytes);
      u32x4 buf[kVecPerLane];
#pragma unroll
      for (int k = 0; k < kVecPerLane; ++k) buf[k] = vp[lane + kWave * k];
#pragma unroll
      for (int k = 0; k < kVecPerLane; ++k) {
        float z[E::kPerVec];
        E::unpack(buf[k], z);
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e) take(z[e]);
      }
    } else if (!kVec) {  // split at 16-byte boundaries; the -inf padding past the body is not taken
      u32x4 buf[kVecPerLane];
      const SplitEdge se = load_split_chunk<E>(rp, c0, n, lane, buf);
#pragma unroll
      for (int k = 0; k < kVecPerLane; ++k) {
        float z[E::kPerVec];
        E::unpack(buf[k], z);
        if (lane + kWave * k < se.body) {
#pragma unroll
          for (int e = 0; e < E::kPerVec; ++e) take(z[e]);
        }
      }
      if (se.ok) take(se.z);
    } else {
      for (int32_t v = c0 + lane; v < c0 + n; v += kWave) take(E::at(rp, v));
    }
    acc = wave_sum(acc);
    cp = wave_sum_u32(cp);
    if (lane == 0) {
      strict[c] = acc;
      copies[c] = cp;
    }
  }
}

// The truncation profile of a row slot's request (SDCP "Session Contract"), by a whole wave.
struct RowProfile {
  bool target;
  int32_t row, i;
  float k2;
  int32_t top_k, milli;
  bool by_k, by_p;
};
__device__ __forceinline__ RowProfile row_profile(const Params& P, int32_t slot) {
  RowProfile f;
  f.target = slot < P.n_t;
  f.row = f.target ? slot : slot - P.n_t;
  f.i = request_of_row_wave(P.cu, P.B, f.row, f.target, (int)(threadIdx.x & (kWave - 1)));
  f.k2 = P.temp_each ? k2_of(temperature_of(P.temp_each, f.i)) : P.k2;
  f.top_k = P.top_k ? P.top_k[f.i] : 0;
  f.milli = P.top_p_milli ? P.top_p_milli[f.i] : 1000;
  const bool valid = f.top_k >= 0 && f.milli >= 0 && f.milli <= 1000;
  f.by_k = valid && f.top_k > 0 && f.top_k < P.V;
  f.by_p = valid && f.milli < 1000;
  return f;
}

// The last steps of a row's cut, by one wave: the kept copies of the cut value per chunk in token
// order, each chunk record's mass rewritten to the mass of the chunk's kept tokens, and the token id
// of the last kept copy (unless every copy is kept: chunk cstar is loaded whole and searched in
// registers, its vectors in token order, vector k * 64 + lane; a chunk off the 16-byte grid is
// split, its head elements searched before the vectors and its tail after).  chunks(cb, st, cp), called by
// every lane, gives chunk cb + lane's mass of kept tokens strictly above kappa (in its record's
// frame) and its copies of kappa (0 past the last chunk).  Writes cuts[slot] and kept_tokens[slot].
template <class E, bool kVec, class ChunkFn>
__device__ __forceinline__ void finish_cut(const Params& P, int32_t slot, const char* rp, float2* rec, float kappa,
                                           float k2, uint32_t ties, uint32_t n_eq, int32_t kept, ChunkFn chunks,
                                           int lane) {
  uint32_t carry = 0u;
  int32_t cstar = -1;
  uint32_t rstar = 0u;
  for (int32_t cb = 0; cb < P.C; cb += kWave) {
    const int32_t c = cb + lane;
    float strict_c = 0.0f;
    uint32_t here = 0u;
    chunks(cb, strict_c, here);
    const uint32_t incl = wave_inclusive_scan(here);
    const uint32_t before = carry + incl - here;
    const uint32_t keep_here = n_eq > before ? min(n_eq - before, here) : 0u;
    if (c < P.C) {
      float s2 = strict_c;
      if (keep_here > 0u && kappa > -INFINITY) s2 += (float)keep_here * fast_exp2(fmaf(kappa, k2, -rec[c].x));
      rec[c].y = s2;
    }
    const uint64_t holds = __ballot(c < P.C && before < n_eq && n_eq <= before + here);
    if (holds && cstar < 0) {
      const int g = __ffsll((unsigned long long)holds) - 1;
      cstar = cb + g;
      rstar = lane_value(n_eq - before, g);
    }
    carry += lane_value(incl, kWave - 1);
  }
  int32_t vcut = INT32_MAX;
  if (n_eq < ties && cstar >= 0) {
    const int32_t c0 = cstar * E::kChunk, end = min(c0 + E::kChunk, P.V);
    uint32_t need = rstar;
    u32x4 buf[kVecPerLane];
    int32_t b0 = c0, nb = (end - c0) / E::kPerVec;  // the first vector element; vectors
    SplitEdge se{};
    if constexpr (kVec) {
      load_chunk<E>(rp, c0, end - c0, lane, buf);
    } else {  // split at 16-byte boundaries: the head's elements, the vectors, the tail's elements
      se = load_split_chunk<E>(rp, c0, end - c0, lane, buf);
      b0 = c0 + se.head;
      nb = se.body;
    }
    // the need-th copy among the lanes flagged by hit (in lane order), if there are that many
    auto among = [&](bool hit, int32_t v) {
      const uint64_t m = __ballot(hit);
      const uint32_t total = (uint32_t)__popcll((unsigned long long)m);
      if (need > total) {
        need -= total;
        return false;
      }
      uint64_t mm = m;
      for (uint32_t q = 1; q < need; ++q) mm &= mm - 1;  // drop the first need - 1 hits
      vcut = lane_value(v, __ffsll((unsigned long long)mm) - 1);
      return true;
    };
    bool found = !kVec && among(se.ok && lane < se.head && se.z == kappa, se.v);
    // no break: a loop left early is not unrolled, and its indexing would put buf in scratch memory
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) {
      if (found) continue;
      float z[E::kPerVec];
      E::unpack(buf[k], z);
      uint32_t mask = 0u;
#pragma unroll
      for (int e = 0; e < E::kPerVec; ++e)
        if (lane + kWave * k < nb && z[e] == kappa) mask |= 1u << e;
      const uint32_t mine = (uint32_t)__popc(mask);
      const uint32_t incl = wave_inclusive_scan(mine);
      const uint32_t total = lane_value(incl, kWave - 1);
      if (need <= total) {
        const uint64_t at = __ballot(incl - mine < need && need <= incl);
        const int g = __ffsll((unsigned long long)at) - 1;
        int32_t v = -1;
        uint32_t left = need - (incl - mine);
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e)
          if ((mask >> e) & 1u) {
            if (left == 1u && v < 0) v = b0 + (lane + kWave * k) * E::kPerVec + e;
            --left;
          }
        vcut = lane_value(v, g);
        found = true;
      } else {
        need -= total;
      }
    }
    if (!kVec && !found) among(se.ok && lane >= se.head && se.z == kappa, se.v);
  }
  if (lane == 0) {
    P.cuts[slot] = Cut{kappa, vcut};
    if (P.kept_tokens) P.kept_tokens[slot] = kept;
  }
}

// The cut of one row slot by a workgroup of kCutThreads.  Rows of requests that sample with a
// profile that truncates get their cut; every other row gets the trivial one.  Writes cuts[slot],
// kept_tokens[slot] and, for a truncated row, the masses of its chunk records.
template <class E, bool kVec>
__device__ __forceinline__ void cut_row(const Params& P, int32_t slot, unsigned char* smem, CutShared& sh) {
  const int t = threadIdx.x, lane = t & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const RowProfile f = row_profile(P, slot);
  const float k2 = f.k2;
  const bool by_k = f.by_k, by_p = f.by_p;
  const int32_t top_k = f.top_k, milli = f.milli;
  auto untruncated = [&]() {
    if (t == 0) {
      P.cuts[slot] = Cut{-INFINITY, INT32_MAX};
      if (P.kept_tokens) P.kept_tokens[slot] = P.V;
    }
  };
  // greedy or rejected requests, and profiles that truncate nothing (the draft rows of greedy
  // requests have no records: they are never read)
  if (!(k2 > 0.0f) || !(by_k || by_p)) return untruncated();
  float2* rec = P.part + (int64_t)slot * P.C;
  // the row's exponent reference R: the largest chunk reference (fl(max z * k))
  float rl = -INFINITY;
  for (int32_t c = t; c < P.C; c += kCutThreads) rl = fmaxf(rl, rec[c].x);
  rl = wave_max(rl);
  if (lane == 0) sh.wave_ref[wave] = rl;
  __syncthreads();
  float R = -INFINITY;
  for (int w = 0; w < kCutWaves; ++w) R = fmaxf(R, sh.wave_ref[w]);
  __syncthreads();
  if (R == -INFINITY) return untruncated();  // a row of -inf only describes no distribution
  const char* rp = f.target ? row_ptr<E>(P.target, f.row, P.V) : row_ptr<E>(P.draft, f.row, P.V);

  Selected s{0u, 0u, 0ull, 0u};
  uint32_t n_eq = 0u;  // copies of the cut value that are kept
  bool done = false;
  uint32_t* top_cnt = (E::kBytes == 2 && P.C <= kTopChunks) ? reinterpret_cast<uint32_t*>(smem + 16 * 1024) : nullptr;
  uint32_t top = 0u;
  if constexpr (E::kBytes == 2) {
    // the 4096 keys below one just above the row maximum's (R = fl(max z * k), whose quotient by k
    // lies within a rounding step of the maximum)
    const uint32_t k_hat = key16_of_bits(__float_as_uint(R / k2) >> 16);
    top = k_hat + 4u > 65535u ? 65535u : k_hat + 4u;
    const uint32_t bottom = top >= (uint32_t)(kRegionKeys - 1) ? top - (uint32_t)(kRegionKeys - 1) : 0u;
    uint32_t* cnt = reinterpret_cast<uint32_t*>(smem);
    done = window_count<kVec>(rp, P.V, P.C, top, bottom, cnt, top_cnt, sh) &&
           window_pick(cnt, top, bottom, P.C, rec, k2, R, by_k, top_k, by_p, milli, sh, s, n_eq);
  }
  __syncthreads();
  if (!done) radix_select<E, kVec>(rp, P.V, k2, R, by_k, top_k, by_p, milli, smem, sh, s, n_eq);
  const float kappa = key_logit(s.key);
  const int32_t kept = (int32_t)(s.cnt_above + n_eq);

  // chunk masses of the kept tokens strictly above the cut value, and the copies of the cut value
  // in each chunk: from the window's per-chunk counts when every kept key is among them (no second
  // read of the row), else by a pass over the row (the histograms' LDS is free again)
  __syncthreads();
  const bool from_counts = done && top_cnt && top - (s.key >> 16) < (uint32_t)kTopKeys;
  float* strict = reinterpret_cast<float*>(smem);
  uint32_t* copies = reinterpret_cast<uint32_t*>(smem + (from_counts ? 8 * 1024 : 16 * 1024));
  if (from_counts) {
    const uint32_t kkey = s.key >> 16;
    for (int32_t c = wave; c < P.C; c += kCutWaves) {
      const float ref_c = rec[c].x;
      float acc = 0.0f;
      uint32_t cp = 0u;
      for (int j = lane; j < kTopKeys && j <= (int)top; j += kWave) {
        const uint32_t key = top - (uint32_t)j, n = top_cnt[c * kTopKeys + j];
        if (n && key > kkey) acc += (float)n * fast_exp2(fmaf(key_logit(key16_to_key(key)), k2, -ref_c));
        if (key == kkey) cp = n;
      }
      acc = wave_sum(acc);
      cp = wave_sum_u32(cp);
      if (lane == 0) {
        strict[c] = acc;
        copies[c] = cp;
      }
    }
  } else {
    chunk_pass<E, kVec>(rp, P.V, P.C, rec, kappa, k2, strict, copies, lane, wave);
  }
  __syncthreads();
  if (wave == 0)
    finish_cut<E, kVec>(P, slot, rp, rec, kappa, k2, s.ties, n_eq, kept,
                        [&](int32_t cb, float& st, uint32_t& cp) {
                          const int32_t c = cb + lane;
                          st = c < P.C ? strict[c] : 0.0f;
                          cp = c < P.C ? copies[c] : 0u;
                        },
                        lane);
  __syncthreads();  // the shared memory is free for the next row
}

// Full cuts: one workgroup per row slot (target rows, then draft rows when the draft side is
// logits), or (kPending), after the count kernel, one per row it left pending (workgroup k takes
// the k-th; the others end at once).
template <class E, bool kVec, bool kPending>
__global__ __launch_bounds__(kCutThreads) void row_cuts(Params P) {
  __shared__ __align__(16) unsigned char smem[48 * 1024];
  __shared__ CutShared sh;
  if constexpr (kPending) {
    // the list is uniform: saying so keeps the row's addressing scalar
    if ((int32_t)blockIdx.x < P.pending[0])
      cut_row<E, kVec>(P, __builtin_amdgcn_readfirstlane(P.pending[1 + blockIdx.x]), smem, sh);
  } else {
    cut_row<E, kVec>(P, (int32_t)blockIdx.x, smem, sh);
  }
}

// The count kernel: one wave per row slot of a truncating bf16 call whose row pass counted, per
// chunk, the kHistKeys keys at and below the chunk maximum's.  Every chunk's window covers the
// row's top kHistKeys keys (no chunk maximum lies above the row maximum), so their counts are the
// sums of the chunks' counts.  When the cut of top-k, then top-p, lands among them it follows from
// the counts alone (the same selection as the window's), and so do the kept masses of the chunks;
// the row is read only where ties of the cut value leave a token id to find.  Otherwise (the cut
// lies deeper, or a chunk that could not be counted reaches the window) the row is left pending
// for row_cuts.  Lane l holds the keys top - 2l and top - 2l - 1.
template <bool kVec>
__global__ __launch_bounds__(256) void row_cuts_counted(Params P) {
  // per wave: the lanes' contributions to 16 chunks, transposed (rows padded to 65 words), and
  // the 64 chunk sums of a batch
  constexpr int kTr = 16, kTrStride = kWave + 1;
  __shared__ float tr_mass[4][kTr * kTrStride];
  __shared__ uint32_t tr_copies[4][kTr * kTrStride];
  __shared__ float sum_mass[4][kWave];
  __shared__ uint32_t sum_copies[4][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int64_t slot64 = (int64_t)blockIdx.x * 4 + wave;
  const int64_t rows = P.qrows ? P.n_t : (int64_t)P.n_t + P.n_d;
  if (slot64 >= rows) return;
  const int32_t slot = (int32_t)slot64;
  const RowProfile f = row_profile(P, slot);
  auto write_cut = [&](Cut c, int32_t kept) {
    if (lane == 0) {
      P.cuts[slot] = c;
      if (P.kept_tokens) P.kept_tokens[slot] = kept;
    }
  };
  auto leave_pending = [&]() {
    if (lane == 0) P.pending[1 + atomicAdd(&P.pending[0], 1)] = slot;
  };
  if (!(f.k2 > 0.0f) || !(f.by_k || f.by_p)) return write_cut(Cut{-INFINITY, INT32_MAX}, P.V);
  float2* rec = P.part + (int64_t)slot * P.C;
  const uint32_t* htop = P.hist_top + (int64_t)slot * P.C;
  const uint16_t* hist = reinterpret_cast<const uint16_t*>(P.hist) + (int64_t)slot * P.C * kHistKeys;
  // R (the largest chunk reference), the row's top key and whether an uncounted chunk reaches it
  float R = -INFINITY;
  uint32_t top = 0u;
  for (int32_t c = lane; c < P.C; c += kWave) {
    R = fmaxf(R, rec[c].x);
    top = max(top, htop[c] & 0xffffu);
  }
  R = wave_max(R);
  top = wave_max_u32(top);
  if (R == -INFINITY) return write_cut(Cut{-INFINITY, INT32_MAX}, P.V);  // a row of -inf only
  bool bad = false;
  for (int32_t c = lane; c < P.C; c += kWave)
    bad |= (htop[c] & kNoCounts) && (htop[c] & 0xffffu) + (uint32_t)kHistKeys > top;
  if (__ballot(bad)) return leave_pending();
  const int j0 = 2 * lane;
  // the counts of keys top - j0 and top - j0 - 1 in chunks cb + q0 .. cb + q0 + kBatch - 1 of the
  // batch of 64 whose tops the lanes hold (mine), loaded before any is used
  constexpr int kBatch = 16;
  auto load_counts = [&](int32_t cb, int q0, int nc, uint32_t mine, uint32_t (&a)[kBatch], uint32_t (&b)[kBatch]) {
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      a[r] = b[r] = 0u;
      const int q = q0 + r;
      const uint32_t tq = q < nc ? (uint32_t)__builtin_amdgcn_readlane((int)mine, q) : kNoCounts;
      if (tq & kNoCounts) continue;  // an uncounted chunk lies wholly below the window
      const int d = j0 - (int)(top - tq);  // chunk-local index of key top - j0
      const uint16_t* hc = hist + (int64_t)(cb + q) * kHistKeys;
      if (d >= 0 && d < kHistKeys) a[r] = hc[d];
      if (d + 1 >= 0 && d + 1 < kHistKeys) b[r] = hc[d + 1];
    }
  };
  // summed over the chunks; rows of at most kBatch chunks keep their counts for the chunk masses
  uint32_t n0 = 0u, n1 = 0u;
  uint32_t a_held[kBatch], b_held[kBatch];
  for (int32_t cb = 0; cb < P.C; cb += kWave) {
    const uint32_t mine = cb + lane < P.C ? htop[cb + lane] : kNoCounts;
    const int nc = min(kWave, P.C - cb);
    for (int q0 = 0; q0 < nc; q0 += kBatch) {
      load_counts(cb, q0, nc, mine, a_held, b_held);
#pragma unroll
      for (int r = 0; r < kBatch; ++r) {
        n0 += a_held[r];
        n1 += b_held[r];
      }
    }
  }
  const uint32_t key0 = top - (uint32_t)j0, key1 = key0 - 1u;
  const uint64_t e0 = fixed_mass(key_logit(key16_to_key(key0)), f.k2, R);
  const uint64_t e1 = fixed_mass(key_logit(key16_to_key(key1)), f.k2, R);
  const uint64_t m0 = f.by_p ? (uint64_t)n0 * e0 : 0ull, m1 = f.by_p ? (uint64_t)n1 * e1 : 0ull;
  // inclusive scans over the lanes (rank order) of the counts and masses
  uint32_t ci = n0 + n1;
  uint64_t mi = m0 + m1;
  ci = wave_inclusive_scan(ci);
  mi = wave_inclusive_scan(mi);
  const uint32_t c_before = ci - n0 - n1;
  const uint64_t m_before = mi - m0 - m1;
  // the key at which a selection lands, by its lane: (key, count above, mass above, copies)
  auto land = [&](bool at0, bool at1, Selected& out) {
    const uint64_t who = __ballot(at0 || at1);
    if (!who) return false;
    const int g = __ffsll((unsigned long long)who) - 1;
    const bool first = at0;
    const uint32_t key = lane_value(first ? key0 : key1, g);
    const uint32_t above = lane_value(first ? c_before : c_before + n0, g);
    const uint64_t mass = lane_value(first ? m_before : m_before + m0, g);
    const uint32_t ties = lane_value(first ? n0 : n1, g);
    out = Selected{key16_to_key(key), above, mass, ties};
    return true;
  };
  Selected s{0u, 0u, 0ull, 0u};
  uint32_t n_eq = 0u;
  uint64_t mass_k = 0ull;
  if (f.by_k) {
    const uint32_t need = (uint32_t)f.top_k;
    if (!land(c_before < need && need <= c_before + n0, c_before + n0 < need && need <= ci, s))
      return leave_pending();  // the top-k cut lies below the window
    n_eq = need - s.cnt_above;
    mass_k = s.mass_above + (uint64_t)n_eq * fixed_mass(key_logit(s.key), f.k2, R);
  } else if (f.by_p) {
    // the row's mass in fixed point, from the chunk records (fp64 across chunks)
    double part = 0.0;
    for (int32_t c = lane; c < P.C; c += kWave)
      if (rec[c].y > 0.0f) part += (double)rec[c].y * exp2((double)rec[c].x - (double)R);
    mass_k = (uint64_t)(wave_sum(part) * (double)kFixScale);
  }
  if (f.by_p) {
    // the first key (rank order) where the running mass reaches the nucleus mass
    const double target = (double)mass_k * ((double)f.milli / 1000.0);
    Selected sp;
    if (!land(n0 > 0u && (double)(m_before + m0) >= target, n1 > 0u && (double)(mi) >= target, sp))
      return leave_pending();  // the nucleus reaches below the window
    uint32_t n = copies_to_reach(sp.mass_above, fixed_mass(key_logit(sp.key), f.k2, R), sp.ties, target);
    if (f.by_k && sp.key == s.key && n > n_eq) n = n_eq;
    s = sp;
    n_eq = n;
  }
  const float kappa = key_logit(s.key);
  const int32_t kept = (int32_t)(s.cnt_above + n_eq);
  const char* rp = f.target ? row_ptr<Bf16>(P.target, f.row, P.V) : row_ptr<Bf16>(P.draft, f.row, P.V);
  const uint32_t kkey = s.key >> 16;
  // per chunk: the kept mass above kappa (in the chunk record's frame) and the copies of kappa,
  // from the chunk's counts of the lanes' keys (a second pass over counts that are still cached)
  const float z0 = key_logit(key16_to_key(key0)), z1 = key_logit(key16_to_key(key1));
  finish_cut<Bf16, kVec>(P, slot, rp, rec, kappa, f.k2, s.ties, n_eq, kept,
                         [&](int32_t cb, float& st, uint32_t& cp) {
                           const int nc = min(kWave, P.C - cb);
                           const uint32_t mine = cb + lane < P.C ? htop[cb + lane] : kNoCounts;
                           const float mine_ref = cb + lane < P.C ? rec[cb + lane].x : 0.0f;
                           for (int q0 = 0; q0 < nc; q0 += kTr) {
                             // this lane's two keys in chunks cb + q0 .. cb + q0 + 15: row r of the
                             // transposed block holds chunk q0 + r, column l lane l's share
                             static_assert(kTr == kBatch, "one batch of counts per transposed block");
                             {
                               constexpr int h = 0;
                               uint32_t a[kBatch], b[kBatch];
                               if (P.C <= kBatch) {  // the counts summed above, still in registers
#pragma unroll
                                 for (int r = 0; r < kBatch; ++r) {
                                   a[r] = a_held[r];
                                   b[r] = b_held[r];
                                 }
                               } else {
                                 load_counts(cb, q0, nc, mine, a, b);
                               }
#pragma unroll
                               for (int r = 0; r < kBatch; ++r) {
                                 const int q = q0 + h + r;
                                 const float ref_q =
                                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine_ref), q < nc ? q : 0));
                                 float m = 0.0f;
                                 if (a[r] && key0 > kkey) m += (float)a[r] * fast_exp2(fmaf(z0, f.k2, -ref_q));
                                 if (b[r] && key1 > kkey) m += (float)b[r] * fast_exp2(fmaf(z1, f.k2, -ref_q));
                                 tr_mass[wave][(h + r) * kTrStride + lane] = m;
                                 tr_copies[wave][(h + r) * kTrStride + lane] = key0 == kkey ? a[r] : (key1 == kkey ? b[r] : 0u);
                               }
                             }
                             __builtin_amdgcn_wave_barrier();  // a wave's shared-memory operations complete in order
                             if (lane < kTr && q0 + lane < nc) {  // lane r sums row r in lane order
                               float m = 0.0f;
                               uint32_t e = 0u;
                               for (int l = 0; l < kWave; ++l) {
                                 m += tr_mass[wave][lane * kTrStride + l];
                                 e += tr_copies[wave][lane * kTrStride + l];
                               }
                               sum_mass[wave][q0 + lane] = m;
                               sum_copies[wave][q0 + lane] = e;
                             }
                             __builtin_amdgcn_wave_barrier();
                           }
                           st = lane < nc ? sum_mass[wave][lane] : 0.0f;
                           cp = lane < nc ? sum_copies[wave][lane] : 0u;
                           __builtin_amdgcn_wave_barrier();
                         },
                         lane);
}

// ============================================================================ 3. verdicts

// Row fold by one wave, lanes over chunks.  T > 0: l2 = R + log2(sum_c s_c 2^(ref_c - R)) with
// R = max_c ref_c.  T = 0: the row argmax (chunk maxima with their first indices; ties to the
// smaller index).
struct RowFold {
  double l2;
  float ref;
  int32_t argmax;
};

template <bool kGreedy>
__device__ __forceinline__ RowFold fold_row(const float2* p, int32_t C, int lane) {
  RowFold f{0.0, -INFINITY, 0};
  if constexpr (kGreedy) {
    float best = -INFINITY;
    int32_t idx = INT32_MAX;
    for (int32_t c = lane; c < C; c += kWave) {
      const float2 r = p[c];
      const int32_t ri = __float_as_int(r.y);
      if (r.x > best || (r.x == best && ri < idx)) {
        best = r.x;
        idx = ri;
      }
    }
    wave_argmax(best, idx);
    f.argmax = idx == INT32_MAX ? 0 : idx;  // a row of -inf only: index 0
  } else {
    float R = -INFINITY;
    for (int32_t c = lane; c < C; c += kWave) R = fmaxf(R, p[c].x);
    R = wave_max(R);
    f.ref = R;
    if (R == -INFINITY) {
      f.l2 = -(double)INFINITY;
      return f;
    }
    double s = 0.0;
    for (int32_t c = lane; c < C; c += kWave) {
      const float2 r = p[c];
      if (r.y > 0.0f) s += (double)r.y * exp2((double)r.x - (double)R);
    }
    f.l2 = (double)R + log2(wave_sum(s));
  }
  return f;
}

// The T > 0 fold of a row of at most 16 (32) chunks by one row of 16 lanes (one half wave): lane c
// holds chunk c, or (-inf, 0) past the last; four (two) rows per wave.  The same values as
// fold_row: there the other lanes only add +0 to the sum and -inf to the maximum.
template <int kLanes>
__device__ __forceinline__ RowFold fold_row_narrow(float2 r) {
  static_assert(kLanes == 16 || kLanes == 32, "a row of 16 lanes or a half wave");
  RowFold f{0.0, -INFINITY, 0};
  const float R = kLanes == 16 ? row16_max(r.x) : half_max(r.x);
  f.ref = R;
  const double s = r.y > 0.0f ? (double)r.y * exp2((double)r.x - (double)R) : 0.0;
  f.l2 = (double)R + log2(kLanes == 16 ? row16_sum(s) : half_sum(s));  // a row of -inf only: -inf
  return f;
}

__device__ __forceinline__ void write_reject(const Params& P, int32_t i, int32_t trow0, int K, bool write_slots, int lane) {
  if (write_slots)
    for (int j = lane; j <= K; j += kWave) P.out_tokens[trow0 + j] = -1;
  if (lane == 0) {
    P.accepted_len[i] = -1;
    if (P.emitted_len) P.emitted_len[i] = 0;
    if (P.dg.terminal_kind) P.dg.terminal_kind[i] = SDV_TERM_BAD;
  }
}

// Request i's stop list [s0, s1) lies inside the stop-token array (or there is none).
__device__ __forceinline__ bool stop_list_valid(const Params& P, int32_t i) {
  if (!P.stop_off) return true;
  const int64_t s0 = P.stop_off[i], s1 = P.stop_off[i + 1];
  return s0 >= 0 && s1 >= s0 && s1 <= P.n_stop;
}

// How many of the a + 1 candidate tokens (the accepted drafts x_0 .. x_{a-1} in lanes 0 .. a-1,
// then the extra token) are emitted: none after the first stop token and no more than the
// remaining budget (SDCP "Verification and Commit", step 7; M7.8 section 0x09).  The extra token
// is emitted only when the count reaches a + 1, so the answer is known before it is drawn.
// Wave-uniform result.
__device__ __forceinline__ int emitted_count(const Params& P, int32_t i, int32_t x, int a, int lane) {
  int n = a + 1;
  if (P.stop_off) {
    bool hit = false;
    const int32_t s0 = P.stop_off[i], s1 = P.stop_off[i + 1];
    for (int32_t s = s0; s < s1; ++s) hit |= lane < a && x == P.stop_tok[s];
    const uint64_t m = __ballot(hit);
    if (m) n = __ffsll((unsigned long long)m);  // the first stop among the drafts, inclusive
  }
  if (P.budget) n = min(n, max(P.budget[i], 0));
  return n;
}

// Decision of wave 0, shared with the other waves of the workgroup.
struct Decision {
  int32_t kind;  // sdv_terminal_kind, SDV_TERM_BAD when the request is rejected
  int32_t a;
  float ref_t, e_hi, q_scale;
  double u;
  double l2_t;   // base-2 LSE of the drawn target row: weights in the frame 2^(z k - ref_t) sum to 2^(l2_t - ref_t)
  Cut ct, cd;  // cuts of the drawn position's target and draft rows (truncating profiles)
};

template <class E, bool kVec, bool kQ, bool kCut, int kWaves>
__device__ __forceinline__ void draw_terminal(const Params& P, const Decision d, float k2, int32_t i, int32_t trow0,
                                              int32_t drow0, const float2* rec_t, double* lds_mass, int lane,
                                              int wave, int n_waves);

static_assert(kVecPerLane % 16 == 0, "the in-chunk search gives each wave (8 or 16) whole rows of 64 vectors");
constexpr int kMaxRows = 2 * SDV_MAX_DEPTH + 1;

// Folds a request's rows: rows r <= K_t are its target rows r (records at rec_t), rows r > K_t its
// draft rows j = r - K_t - 1 (records at draft_rec(j)).  All chunk records go to shared memory in one
// pass when they fit the budget (else the fold reads the workspace); `overlap` runs between the
// staging loads and the barrier (wave 0's gathers hide under them).  rows[r] receives the fold of row r.
template <bool kGreedy, class DraftRec, class Overlap>
__device__ __forceinline__ void stage_and_fold(const Params& P, const float2* rec_t, DraftRec draft_rec, int K_t,
                                               int n_rows, double* lds_mass, RowFold* rows, int lane, int wave,
                                               int n_waves, Overlap overlap) {
  const int64_t n_rec = (int64_t)n_rows * P.C;
  float2* lds_rec = reinterpret_cast<float2*>(lds_mass + P.C);
  const bool staged = n_rec <= P.lds_records;
  if (staged) {
    for (int64_t q = threadIdx.x; q < n_rec; q += blockDim.x) {
      const int64_t r = q / P.C;
      const int32_t c = (int32_t)(q - r * P.C);
      lds_rec[q] = r <= K_t ? rec_t[r * P.C + c] : draft_rec((int)(r - K_t - 1))[c];
    }
  }
  overlap();
  __syncthreads();
  auto records_of = [&](int r) {
    return staged ? lds_rec + (int64_t)r * P.C
                  : (r <= K_t ? rec_t + (int64_t)r * P.C : draft_rec(r - K_t - 1));
  };
  auto fold_narrow = [&](auto lanes) {  // kWave / lanes rows per wave
    constexpr int kLanes = decltype(lanes)::value, kPer = kWave / kLanes;
    const int g = lane / kLanes, c = lane % kLanes;
    for (int r0 = kPer * wave; r0 < n_rows; r0 += kPer * n_waves) {
      const int r = r0 + g;
      const float2 rec = r < n_rows && c < P.C ? records_of(r)[c] : make_float2(-INFINITY, 0.0f);
      const RowFold f = fold_row_narrow<kLanes>(rec);
      if (c == 0 && r < n_rows) rows[r] = f;
    }
  };
  if (!kGreedy && P.C <= 16) {
    fold_narrow(std::integral_constant<int, 16>{});
  } else if (!kGreedy && P.C <= 32) {
    fold_narrow(std::integral_constant<int, 32>{});
  } else {
    for (int r = wave; r < n_rows; r += n_waves) {
      const RowFold f = fold_row<kGreedy>(records_of(r), P.C, lane);
      if (lane == 0) rows[r] = f;
    }
  }
  __syncthreads();
}

// The verdict of request i under one rule (k2 = log2(e)/T and the Philox key seed), by one
// workgroup of 8 waves.  Shared memory: the folded rows, the decision, and the residual chunk masses
// (C doubles, dynamic).  bad_profile rejects the request once its offsets have been screened.  With
// kCut the rows' cuts (top-k / top-p) decide which tokens p and q keep; the chunk records already
// hold the kept masses.  With P.split workgroups per request (blockIdx.y = 0 .. split - 1) every
// one reaches the same decision from the same loads; the first writes it, and a correction's
// residual pass is shared among them (draw_terminal).
template <class E, bool kGreedy, bool kVec, bool kQ, bool kCut, int kWaves>
__device__ __forceinline__ void verdict_body(const Params& P, int32_t i, float k2, uint64_t seed, bool bad_profile,
                                             double* lds_mass, RowFold* rows, Decision& dec) {
  const int lane = threadIdx.x & (kWave - 1);
  // the wave index is uniform over the wave; saying so keeps every loop and load condition that
  // depends on it a scalar branch (a lane-predicated load would force a wait for all loads in flight)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n_waves = blockDim.x / kWave;
  const bool lead = blockIdx.y == 0;  // the workgroup that writes the decision
  if constexpr (kGreedy) {
    if (!lead) return;  // nothing to share
  }

  // screening: every wave reaches the same answer from the same loads
  // the request's offsets load beside the batch-wide screening (i < B: both are in bounds)
  const int32_t lo_raw = P.cu[i], hi_raw = P.cu[i + 1];
  const bool ok_offsets = *P.batch_ok != 0;
  const int32_t lo = ok_offsets ? lo_raw : 0, hi = ok_offsets ? hi_raw : 0;
  const int K = hi - lo;
  const int32_t trow0 = lo + i, drow0 = lo;
  if (!ok_offsets || K > SDV_MAX_DEPTH) {  // malformed batch, or the depth limit: no slot written
    if (wave == 0 && lead) write_reject(P, i, 0, 0, false, lane);
    return;
  }
  if (bad_profile || !stop_list_valid(P, i)) {  // no profile, or no stop set: every slot is -1
    if (wave == 0 && lead) write_reject(P, i, trow0, K, true, lane);
    return;
  }
  const float2* rec_t = P.part + (int64_t)trow0 * P.C;
  const float2* rec_d = P.part + (int64_t)(P.n_t + drow0) * P.C;

  // 1. all chunk records of the request's rows (r <= K target row r, r > K draft row r - K - 1)
  // are staged in shared memory in one pass when they fit, while wave 0 fetches the draft
  // tokens and the logits at them
  const int n_rows = (kGreedy || kQ) ? K + 1 : 2 * K + 1;  // given q rows have no records
  const bool active = lane < K;
  int32_t x = 0;
  float zt = 0.0f, zd = 0.0f;
  bool keep_t = true, keep_d = true;  // x is kept by the target / draft row's truncation
  auto draft_rec = [&](int j) { return rec_d + (int64_t)j * P.C; };
  stage_and_fold<kGreedy>(P, rec_t, draft_rec, K, n_rows, lds_mass, rows, lane, wave, n_waves, [&] {
    if (wave == 0 && active) {
      x = P.tokens[drow0 + lane];
      if constexpr (!kGreedy) {
        if (x >= 0 && x < P.V) {
          zt = E::at(row_ptr<E>(P.target, trow0 + lane, P.V), x);
          // with q rows, zd carries q(x) itself
          zd = kQ ? P.qrows[(int64_t)(drow0 + lane) * P.V + x] : E::at(row_ptr<E>(P.draft, drow0 + lane, P.V), x);
          if constexpr (kCut) {
            keep_t = kept_by(P.cuts[trow0 + lane], zt, x);
            if constexpr (!kQ) keep_d = kept_by(P.cuts[P.n_t + drow0 + lane], zd, x);
          }
        }
      }
    }
  });

  // 2. the verdict, by wave 0
  if (wave == 0) {
    Decision d{SDV_TERM_BAD, 0, 0.0f, 0.0f, 0.0f, 0.0, 0.0, Cut{-INFINITY, INT32_MAX}, Cut{-INFINITY, INT32_MAX}};
    if (__ballot(active && (x < 0 || x >= P.V)) != 0) {
      if (lead) write_reject(P, i, trow0, K, true, lane);
    } else if constexpr (kGreedy) {
      const int32_t g = lane <= K ? rows[lane].argmax : 0;
      const uint64_t miss = __ballot(active && x != g);
      const int a = miss ? __ffsll((unsigned long long)miss) - 1 : K;
      const int32_t g_a = rows[a].argmax;
      const int n_emit = emitted_count(P, i, x, a, lane);
      for (int j = lane; j <= K; j += kWave) P.out_tokens[trow0 + j] = j >= n_emit ? -1 : (j < a ? x : g_a);
      if (P.dg.target_argmax)
        for (int j = lane; j <= K; j += kWave) P.dg.target_argmax[trow0 + j] = rows[j].argmax;
      if (lane == 0) {
        P.accepted_len[i] = a;
        if (P.emitted_len) P.emitted_len[i] = n_emit;
        if (P.dg.terminal_kind) P.dg.terminal_kind[i] = n_emit == a + 1 ? SDV_TERM_GREEDY : SDV_TERM_NONE;
      }
      d.kind = SDV_TERM_GREEDY;
    } else {
      RowFold ft{0.0, 0.0f, 0}, fd{0.0, 0.0f, 0};
      double ratio = 0.0;
      double r = 1.0;
      bool qzero = false;
      bool accept = true;
      Philox4 blk{0u, 0u, 0u, 0u};
      if (active) {
        ft = rows[lane];
        if constexpr (kQ) {  // p(x) = 2^(z_t k - l2_t), q(x) given
          qzero = !(zd > 0.0f);
          ratio = exp2((double)zt * (double)k2 - ft.l2) / (double)zd;
        } else {
          fd = rows[K + 1 + lane];
          qzero = zd == -INFINITY || !keep_d;  // a token the draft row does not keep has q = 0
          // log2 p(x)/q(x) = (z_t - z_d) k - (l2_t - l2_d)
          ratio = exp2(((double)zt - (double)zd) * (double)k2 - (ft.l2 - fd.l2));
        }
        if (!keep_t) ratio = 0.0;  // p(x) = 0
        if (P.r_each) {  // the caller's r in [0, 1): SDCP Rule 2, r < p/q
          r = P.r_each[drow0 + lane];
          accept = r < ratio;
        } else {  // Philox r in (0, 1]: r <= p/q
          blk = verifier_block(seed, (uint32_t)i, (uint32_t)lane);
          r = (double)accept_uniform(blk);
          accept = r <= ratio;
        }
      }
      if (__ballot(qzero) != 0) {  // q(x) = 0 somewhere: rejected before any uniform is used
        if (lead) write_reject(P, i, trow0, K, true, lane);
      } else {
        const uint64_t rej = __ballot(active && !accept);
        const int a = rej ? __ffsll((unsigned long long)rej) - 1 : K;
        const int n_emit = emitted_count(P, i, x, a, lane);
        const bool frontier = n_emit == a + 1;
        if (lead) {
          // slot a is written by the draw below when the extra token is emitted
          for (int j = lane; j <= K; j += kWave)
            if (j != a || !frontier) P.out_tokens[trow0 + j] = j < a && j < n_emit ? x : -1;
          if (lane == 0) {
            P.accepted_len[i] = a;
            if (P.emitted_len) P.emitted_len[i] = n_emit;
            if (!frontier && P.dg.terminal_kind) P.dg.terminal_kind[i] = SDV_TERM_NONE;
          }
          if (P.dg.target_lse)
            for (int j = lane; j <= K; j += kWave) P.dg.target_lse[trow0 + j] = rows[j].l2 * kLn2;
          if (active) {
            if (P.dg.draft_lse && !kQ) P.dg.draft_lse[drow0 + lane] = fd.l2 * kLn2;
            if (P.dg.ratio) P.dg.ratio[drow0 + lane] = ratio;
            if (P.dg.accept_uniform) P.dg.accept_uniform[drow0 + lane] = (float)r;
            if (P.dg.target_logit) P.dg.target_logit[drow0 + lane] = zt;
            if (P.dg.draft_logit) P.dg.draft_logit[drow0 + lane] = zd;
          }
        }
        d.a = a;
        if constexpr (kCut) {
          d.ct = P.cuts[trow0 + a];
          d.cd = (!kQ && a < K) ? P.cuts[P.n_t + drow0 + a] : Cut{-INFINITY, INT32_MAX};
        }
        if (!frontier) {  // emission stops inside the accepted drafts: nothing is drawn
          d.kind = SDV_TERM_NONE;
        } else if (a == K) {
          d.kind = SDV_TERM_BONUS;
          d.ref_t = rows[K].ref;
          d.l2_t = rows[K].l2;
          d.u = P.u_each ? P.u_each[trow0 + K] : (double)draw_uniform(verifier_block(seed, (uint32_t)i, (uint32_t)K));
        } else {
          // weights in the frame 2^(z_t k - ref_t) of the rejected target row; draft side
          // 2^(z_d k - e) with e = ref_t + l2_d - l2_t carried as e_hi and the factor 2^-(e - e_hi)
          d.kind = SDV_TERM_RESIDUAL;
          d.ref_t = lane_value(ft.ref, a);
          d.l2_t = lane_value(ft.l2, a);
          if constexpr (kQ) {  // q scaled into the frame: q 2^(l2_t - ref_t)
            d.q_scale = (float)exp2(lane_value(ft.l2, a) - (double)d.ref_t);
          } else {
            const double e = (double)d.ref_t + lane_value(fd.l2, a) - lane_value(ft.l2, a);
            d.e_hi = (float)e;
            d.q_scale = (float)exp2((double)d.e_hi - e);
          }
          d.u = P.u_each ? P.u_each[trow0 + a] : (double)lane_value(draw_uniform(blk), a);
        }
      }
    }
    if (lane == 0) dec = d;
  }
  __syncthreads();
  if constexpr (!kGreedy)
    draw_terminal<E, kVec, kQ, kCut, kWaves>(P, dec, k2, i, trow0, drow0, rec_t, lds_mass, lane, wave, n_waves);
}

// Workgroups (blockIdx.x, s), s < P.split, verify request blockIdx.x.  With a profile per request,
// the request's temperature selects the rule at run time (uniformly over the workgroup).  A top-k
// below 0 or a top-p outside [0, 1000] thousandths describes no profile: the request is rejected
// under either rule.
template <class E, int kMode, bool kVec, bool kQ, bool kCut, int kWaves = kVerdictWaves>
__global__ __launch_bounds__(kWave * kWaves) void verdicts(Params P) {
  extern __shared__ double lds_mass[];  // [C]
  __shared__ RowFold rows[kMaxRows];
  __shared__ Decision dec;
  const int32_t i = blockIdx.x;
  const bool bad_truncation = (P.top_k && P.top_k[i] < 0) ||
                              (P.top_p_milli && (P.top_p_milli[i] < 0 || P.top_p_milli[i] > 1000));
  if constexpr (kMode == kModeProfiled) {
    const float k2 = k2_of(temperature_of(P.temp_each, i));
    const uint64_t seed = P.seed_each[i];
    if (k2 > 0.0f) verdict_body<E, false, kVec, kQ, kCut, kWaves>(P, i, k2, seed, bad_truncation, lds_mass, rows, dec);
    else
      verdict_body<E, true, kVec, false, false, kWaves>(P, i, 0.0f, seed, !(k2 == 0.0f) || bad_truncation, lds_mass,
                                                        rows, dec);
  } else {
    verdict_body<E, kMode == kModeGreedy, kVec, kQ && kMode != kModeGreedy, kCut && kMode != kModeGreedy, kWaves>(
        P, i, P.k2, P.seed, bad_truncation, lds_mass, rows, dec);
  }
}

// A batch of one request whose 16-byte aligned rows hold at most kOneLaunchUnits chunks in all runs
// in one launch of kOneLaunchWaves waves.  Wave w computes the record of chunk w (the row pass's
// work, every chunk at once), the last wave screens the offsets, and the workgroup then verifies
// the request as the verdict kernel does, from the records it has just written (the workgroup
// barrier orders those stores before the loads).  That saves the second launch and the records'
// trip between two kernels.
constexpr int kOneLaunchWaves = 16;
constexpr int64_t kOneLaunchUnits = kOneLaunchWaves - 1;

template <class E, int kMode>
__global__ __launch_bounds__(kWave * kOneLaunchWaves) void one_launch(Params P) {
  static_assert(kMode != kModeProfiled, "one profile per call");
  constexpr bool kVec = true;
  extern __shared__ double lds_mass[];
  __shared__ RowFold rows[kMaxRows];
  __shared__ Decision dec;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (wave == kOneLaunchWaves - 1) screen_offsets(P, lane);
  const int64_t u = wave;
  if (u < P.n_units) {
    const int32_t slot = (int32_t)(u / P.C);
    const int32_t c = (int32_t)(u - (int64_t)slot * P.C);
    const char* rp = slot < P.n_t ? row_ptr<E>(P.target, slot, P.V) : row_ptr<E>(P.draft, slot - P.n_t, P.V);
    const int32_t c0 = c * E::kChunk;
    const float2 rec = chunk_record<E, kMode == kModeGreedy, kVec>(rp, c0, min(E::kChunk, P.V - c0), P.k2, lane);
    if (lane == 0) P.part[u] = rec;
  }
  __syncthreads();  // the records and the screening, seen by every wave
  verdict_body<E, kMode == kModeGreedy, kVec, false, false, kOneLaunchWaves>(P, 0, P.k2, P.seed, false, lds_mass, rows,
                                                                            dec);
}

// The correction or bonus draw of a request (T > 0), by the verdict workgroup.  With P.split
// workgroups per request, workgroup s computes the residual masses of chunks [s C / split,
// (s + 1) C / split) and publishes them; the last one to finish (a counter per request) reads the
// others' and draws.  A bonus draw needs no residual pass: the first workgroup draws it alone.
template <class E, bool kVec, bool kQ, bool kCut, int kWaves>
__device__ __forceinline__ void draw_terminal(const Params& P, const Decision d, float k2, int32_t i, int32_t trow0,
                                              int32_t drow0, const float2* rec_t, double* lds_mass, int lane,
                                              int wave, int n_waves) {
  if (d.kind != SDV_TERM_BONUS && d.kind != SDV_TERM_RESIDUAL) return;  // uniform over the workgroup
  const int32_t n_split = gridDim.y, part = blockIdx.y;
  if (d.kind == SDV_TERM_BONUS && part != 0) return;
  typedef typename std::conditional<kCut, RowCuts, NoCut>::type Mask;
  Mask m{};
  if constexpr (kCut) {  // uniform over the workgroup: scalar registers
    auto uniform = [](Cut c) {
      return Cut{__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c.kappa))),
                 __builtin_amdgcn_readfirstlane(c.vcut)};
    };
    m = RowCuts{uniform(d.ct), uniform(d.cd)};
  }
  const int32_t trow = trow0 + d.a;
  const char* tp = row_ptr<E>(P.target, trow, P.V);
  bool residual = d.kind == SDV_TERM_RESIDUAL;
  const char* dp = residual && !kQ ? row_ptr<E>(P.draft, drow0 + d.a, P.V) : nullptr;
  const float* qp = residual && kQ ? P.qrows + (int64_t)(drow0 + d.a) * P.V : nullptr;

  // a row of one chunk (16-byte aligned logit rows): the in-chunk search totals the weights itself,
  // so neither the mass pass nor the pick of a chunk runs (a split is 1 here: C / 4 < 1); a correction
  // on rows of up to four chunks takes the same single pass over the whole pair when it is not split
  const bool one_chunk = kVec && !kQ && P.C == 1;
  const bool few_chunks = kVec && !kQ && residual && P.C <= 4 && n_split == 1;
  // residual masses of this workgroup's chunks [c_lo, c_hi), into shared memory; the vector passes
  // see the range as a row of its own (tokens from c_lo's first, masks shifted to match)
  const int32_t c_lo = (int32_t)((int64_t)P.C * part / n_split), c_hi = (int32_t)((int64_t)P.C * (part + 1) / n_split);
  const int32_t v_lo = c_lo * E::kChunk, V_r = min(P.V, c_hi * E::kChunk) - v_lo;
  Mask m_r = m;
  if constexpr (kCut) {
    m_r.ct.vcut -= v_lo;
    m_r.cd.vcut -= v_lo;
  }
  if (residual && kQ) {
    for (int32_t c = c_lo + wave; c < c_hi; c += n_waves) {
      const int32_t c0 = c * E::kChunk;
      const double cm = resid_chunk_mass_q_split<E, kVec>(m, tp, qp, P.V, c0, min(E::kChunk, P.V - c0), k2, d.ref_t,
                                                          d.q_scale, lane);
      if (lane == 0) lds_mass[c] = cm;
    }
    __syncthreads();
  } else if (residual && !one_chunk && !few_chunks) {
    if constexpr (kVec && kWaves == kVerdictWaves) {
      resid_masses_pipelined<E>(m_r, tp + (int64_t)v_lo * E::kBytes, dp + (int64_t)v_lo * E::kBytes, V_r,
                                c_hi - c_lo, k2, d.ref_t, d.e_hi, d.q_scale, lds_mass + c_lo, lane, wave, n_waves);
    } else {
      for (int32_t c = c_lo + wave; c < c_hi; c += n_waves) {
        const int32_t c0 = c * E::kChunk;
        const double cm = resid_chunk_mass_split<E, kVec>(m, tp, dp, P.V, c0, min(E::kChunk, P.V - c0), k2, d.ref_t,
                                                          d.e_hi, d.q_scale, lane);
        if (lane == 0) lds_mass[c] = cm;
      }
    }
    __syncthreads();
  }
  if (residual && n_split > 1) {
    // publish this range; the workgroup whose increment completes the count takes every mass.
    // Wave 0 alone stores, fences (device scope: the other workgroups may sit on other XCDs, whose
    // L2s are not coherent with this one's) and counts; nothing waits on another workgroup.
    __shared__ int32_t last;
    if (wave == 0) {
      double* pub = P.split_mass + (int64_t)i * P.Cm;
      for (int32_t c = c_lo + lane; c < c_hi; c += kWave) pub[c] = lds_mass[c];
      __threadfence();
      uint32_t before = 0u;
      if (lane == 0) before = atomicAdd(&P.split_count[(int64_t)i * kLineWords], 1u);
      const bool is_last = lane_value(before, 0) == (uint32_t)(n_split - 1);
      if (is_last) {
        __threadfence();
        for (int32_t c = lane; c < P.C; c += kWave)
          if (c < c_lo || c >= c_hi) lds_mass[c] = pub[c];
      }
      if (lane == 0) last = is_last;
    }
    __syncthreads();
    if (!last) return;
  }
  // S: the total weight of the draw in the frame 2^(z k - ref_t), reported in probability units
  auto write_token = [&](int32_t y, bool empty, double S) {
    if (y >= 0 && lane == 0) {  // the one wave that resolved the token writes it
      P.out_tokens[trow] = y;
      if (P.dg.draw_uniform) P.dg.draw_uniform[i] = (float)d.u;
      if (P.dg.terminal_mass) P.dg.terminal_mass[i] = S * exp2((double)d.ref_t - d.l2_t);
      if (P.dg.terminal_kind)
        P.dg.terminal_kind[i] =
            d.kind == SDV_TERM_BONUS ? SDV_TERM_BONUS : (empty ? SDV_TERM_RESIDUAL_EMPTY : SDV_TERM_RESIDUAL);
    }
  };
  if constexpr (kVec && !kQ) {
    auto single_pass = [&](auto chunks) {
      constexpr int kC = decltype(chunks)::value;
      int32_t y = -1;
      bool empty = false;
      double S = 0.0;
      if (residual) {
        y = search_chunk_block<E, true, true, kC, kWaves>(m, tp, dp, 0, P.V, (double)d.u, k2, d.ref_t, d.e_hi, d.q_scale,
                                                  lds_mass + P.C, lane, wave, n_waves, &S);
        empty = y == -2;  // no positive residual weight in floating point: draw from p_t
        // the fallback search rewrites the row sums every wave has just read: all reads come first
        // (empty is the same in every wave, so the barrier is uniform)
        if (empty) __syncthreads();
      }
      if (!residual || empty)
        y = search_chunk_block<E, false, true, kC, kWaves>(m, tp, nullptr, 0, P.V, (double)d.u, k2, d.ref_t, 0.0f, 0.0f,
                                                   lds_mass + P.C, lane, wave, n_waves, &S);
      write_token(y, empty, S);
    };
    if (one_chunk) return single_pass(std::integral_constant<int, 1>{});
    if (few_chunks) {
      if (P.C == 2) return single_pass(std::integral_constant<int, 2>{});
      return single_pass(std::integral_constant<int, 4>{});
    }
  }
  // every wave picks the same chunk from the same masses
  double S = 0.0;
  if (residual) {
    for (int32_t c = lane; c < P.C; c += kWave) S += lds_mass[c];
    S = wave_sum(S);
  }
  bool empty = false;
  if (residual && !(S > 0.0)) {  // no positive residual weight in floating point: draw from p_t
    residual = false;
    empty = true;
  }
  // a draw from p takes the chunk masses from the row's records (kept masses under truncation)
  const float2* rec = rec_t + (int64_t)d.a * P.C;
  double tgt = 0.0;
  int32_t cs;
  if (residual) {
    cs = pick_chunk(P.C, (double)d.u, [&](int32_t c) { return lds_mass[c]; }, &tgt, &S, lane);
  } else {
    cs = pick_chunk(
        P.C, (double)d.u, [&](int32_t c) { return (double)rec[c].y * exp2((double)rec[c].x - (double)d.ref_t); },
        &tgt, &S, lane);
  }
  const int32_t s0 = cs * E::kChunk;
  const int32_t n = min(E::kChunk, P.V - s0);
  int32_t y = -1;
  if constexpr (kVec) {
    if (residual && kQ)
      y = search_chunk_q_block<E, kWaves>(m, tp, qp, s0, n, tgt, k2, d.ref_t, d.q_scale, lds_mass + P.C, lane, wave,
                                  n_waves);
    else if (residual)
      y = search_chunk_block<E, true, false, 1, kWaves>(m, tp, dp, s0, n, tgt, k2, d.ref_t, d.e_hi, d.q_scale, lds_mass + P.C, lane,
                                      wave, n_waves);
    else
      y = search_chunk_block<E, false, false, 1, kWaves>(m, tp, nullptr, s0, n, tgt, k2, d.ref_t, 0.0f, 0.0f, lds_mass + P.C, lane,
                                       wave, n_waves);
  } else {
    if (residual && kQ) {
      y = search_chunk_q_split<E, kWaves>(m, tp, qp, P.V, s0, n, tgt, k2, d.ref_t, d.q_scale, lds_mass + P.C, lane, wave,
                                  n_waves);
    } else if (residual) {
      y = search_chunk_split<E, true, kWaves>(m, tp, dp, P.V, s0, n, tgt, k2, d.ref_t, d.e_hi, d.q_scale, lds_mass + P.C, lane,
                                      wave, n_waves);
    } else {
      y = search_chunk_split<E, false, kWaves>(m, tp, nullptr, P.V, s0, n, tgt, k2, d.ref_t, 0.0f, 0.0f, lds_mass + P.C,
                                       lane, wave, n_waves);
    }
  }
  write_token(y, empty, S);
}

// ============================================================================ 4. token trees
// Tree verification by multi-step speculative sampling (Miao et al., "SpecInfer", ASPLOS 2024,
// section 4: the token tree verifier).  Request i holds N_i <= 64 nodes; node n has parent
// P.parents[cu[i] + n] in [-1, n - 1] and token P.tokens[cu[i] + n], drawn from the distribution of
// draft row P.draft_row[cu[i] + n] (siblings from one drafter share a row), or of row cu[i] + n.
// Target row cu[i] + i is the root's, cu[i] + i + n + 1 follows node n: the linear layout, so the
// row pass is unchanged and a chain of nodes is a linear draft.
//
// At the current node, with p its target distribution, the children are tested in node order.
// Child c is accepted iff r_c <= p(x_c) / q_c(x_c), r_c from the Philox block (c, i); after l
// rejections p is the residual R_l / M_l, with
//   R_0 = p,  R_j = max(R_{j-1} - M_{j-1} q_{c_j}, 0),  M_j = sum_v R_j(v)  (M_0 = 1),
// the unnormalized form of p <- normalize(max(p - q, 0)) applied j times.  Each rejection costs one
// pass over the node's target row and the rejected children's draft rows (M_j and its chunk
// masses); the extra token is drawn from R_l by those chunk masses and a search inside one chunk,
// or, when no child was rejected, from the node's own target row by its records.  u comes from the
// block of the node's target row.  At T = 0 the first child equal to the node's target argmax is
// accepted.  The walk runs in wave 0; the passes use the whole workgroup.

// Weight R_l(v) in fp32 (probability units): the node's target logit zt and the rejected
// children's draft logits zd[j] at v, exponents carried as (hi, lo) float pairs.
struct ChainFrame {
  int32_t l;                       // rejected children so far
  float k2, t_hi, t_lo;            // the node's target row: log2 p(v) = zt k2 - (t_hi + t_lo)
  float d_hi[SDV_MAX_DEPTH];       // rejected child j's draft row: log2 q(v) = zd k2 - (d_hi + d_lo)
  float d_scale[SDV_MAX_DEPTH];    // 2^(t_lo - d_lo) for child j
  float m[SDV_MAX_DEPTH];          // M_j, the mass before rejection j + 1 (m[0] = 1)
  int32_t drow[SDV_MAX_DEPTH];     // rejected child j's draft row (batch index)
};

// The passes work in units of 2^-t_lo: R'(v) = R(v) 2^t_lo, which starts from 2^(zt k2 - t_hi) and
// takes each draft row's q as 2^(zd k2 - d_hi) with its coefficient scaled by d_scale, so that no
// element pays for the low parts.  Masses summed in these units are scaled back by 2^-t_lo.
__device__ __forceinline__ float chain_p(const ChainFrame& f, float zt) {
  return fast_exp2(fmaf(zt, f.k2, -f.t_hi));
}

// Rejected children j0 .. j1 - 1 share one draft row: its q is loaded and exponentiated once, and
// the run's steps collapse into one, since for q >= 0 and a, b >= 0
// max(max(x - a q, 0) - b q, 0) = max(x - (a + b) q, 0): R = max(R - c q, 0) with c the sum of the
// run's masses M_j (run_mass).
__device__ __forceinline__ int chain_run_end(const ChainFrame& f, int j0) {
  int j1 = j0 + 1;
  while (j1 < f.l && f.drow[j1] == f.drow[j0]) ++j1;
  return j1;
}
__device__ __forceinline__ float run_mass(const ChainFrame& f, int j0, int j1) {
  float c = 0.0f;
  for (int j = j0; j < j1; ++j) c += f.m[j];
  return c * f.d_scale[j0];  // one row: one d_lo for the whole run
}
__device__ __forceinline__ float chain_run(const ChainFrame& f, int j0, int j1, float R, float zd) {
  const float q = fast_exp2(fmaf(zd, f.k2, -f.d_hi[j0]));
  return fmaxf(fmaf(-run_mass(f, j0, j1), q, R), 0.0f);
}

// R_l(v) for one element (rows given as byte pointers of the logits).
template <class E>
__device__ __forceinline__ float chain_weight(const ChainFrame& f, const char* trow, const void* draft, int32_t V,
                                              int32_t v) {
  float R = chain_p(f, E::at(trow, v));
  for (int j = 0; j < f.l;) {
    const int j1 = chain_run_end(f, j);
    R = chain_run(f, j, j1, R, E::at(row_ptr<E>(draft, f.drow[j], V), v));
    j = j1;
  }
  return R;
}

constexpr int kTreeWaves = 16;  // waves of a tree verdict workgroup (the passes are VALU-bound per CU)
constexpr int kTreeGroup = 4;  // vectors per lane in flight per row in a residual pass

// A chunk of a node's target row split on its 16-byte grid for the tree passes, whose draft rows
// each sit at their own offset: while the first vector lies within 16 bytes of the row start it
// joins the head, and while the last ends within 16 bytes of the row end it joins the tail, so the
// two aligned pieces under any vector of any draft row stay inside that row.
struct TreeSplit {
  int32_t head, body;  // elements before the first vector; vectors
  const u32x4* tv;     // target vector j
};
template <class E>
__device__ __forceinline__ TreeSplit tree_split(const char* tp, int32_t V, int32_t c0, int32_t n) {
  const split::Plan p = split::tree((uintptr_t)tp, E::kBytes, V, c0, n);
  return TreeSplit{p.head, p.body, reinterpret_cast<const u32x4*>(at_address(tp, p.first))};
}

// The bytes of draft row dp under body vector jc of a tree split (0 <= jc < body).
template <class E>
__device__ __forceinline__ u32x4 tree_draft_vec(const char* dp, int32_t c0, const TreeSplit& s, int jc) {
  uintptr_t pieces;
  uint32_t shift;
  split::tree_pieces(split::Plan{s.head, s.body, 0u, 0, 0}, (uintptr_t)dp, E::kBytes, c0, &pieces, &shift);
  const u32x4* dv = reinterpret_cast<const u32x4*>(at_address(dp, pieces));
  return funnel16(dv[jc], dv[shift != 0 ? jc + 1 : jc], shift);
}

// Chunk masses of R_l into lds_mass[0 .. C) by the whole workgroup (wave w takes chunks w,
// w + n_waves, ...): 16-byte vectors, four in flight per lane, fp32 per vector, fp64 across vectors
// (rows off the 16-byte grid: split as tree_split says, the edge elements one per lane).
template <class E, bool kVec>
__device__ __forceinline__ void chain_masses(const ChainFrame& f, const char* trow, const void* draft, int32_t V,
                                             int32_t C, double* lds_mass, int lane, int wave, int n_waves) {
  for (int32_t c = wave; c < C; c += n_waves) {
    const int32_t c0 = c * E::kChunk, n = min(E::kChunk, V - c0);
    double acc = 0.0;
    if constexpr (kVec) {
      const int32_t nvec = n / E::kPerVec;
      const u32x4* tv = reinterpret_cast<const u32x4*>(trow + (int64_t)c0 * E::kBytes);
      constexpr int kGroup = kTreeGroup;
      // a full chunk indexes its vectors directly; the partial last one clamps indices into the
      // chunk, which keeps every load unconditional (a vector past the end has a target of -inf, so
      // R is 0 there whatever the draft row holds)
      auto pass = [&](auto full_chunk) {
        constexpr bool kFull = decltype(full_chunk)::value;
        for (int g0 = 0; g0 < kVecPerLane && (kFull || g0 * kWave < nvec); g0 += kGroup) {
          float R[kGroup][E::kPerVec];
          auto jc = [&](int k) { return kFull ? lane + kWave * (g0 + k) : min(lane + kWave * (g0 + k), nvec - 1); };
#pragma unroll
          for (int k = 0; k < kGroup; ++k) {
            const u32x4 t = tv[jc(k)];
            float z[E::kPerVec];
            E::unpack(kFull || lane + kWave * (g0 + k) < nvec ? t : neg_inf_vec<E>(), z);
#pragma unroll
            for (int e = 0; e < E::kPerVec; ++e) R[k][e] = chain_p(f, z[e]);
          }
          for (int j = 0; j < f.l;) {  // one load and one exponential per run of rejections on one row
            const int j1 = chain_run_end(f, j);
            const u32x4* dv =
                reinterpret_cast<const u32x4*>(row_ptr<E>(draft, f.drow[j], V) + (int64_t)c0 * E::kBytes);
            u32x4 b[kGroup];
#pragma unroll
            for (int k = 0; k < kGroup; ++k) b[k] = dv[jc(k)];
            const float d_hi = f.d_hi[j];
            float q[kGroup][E::kPerVec];
#pragma unroll
            for (int k = 0; k < kGroup; ++k) {
              float z[E::kPerVec];
              E::unpack(b[k], z);
#pragma unroll
              for (int e = 0; e < E::kPerVec; ++e) q[k][e] = fast_exp2(fmaf(z[e], f.k2, -d_hi));
            }
            const float cm = run_mass(f, j, j1);
#pragma unroll
            for (int k = 0; k < kGroup; ++k)
#pragma unroll
              for (int e = 0; e < E::kPerVec; ++e) R[k][e] = fmaxf(fmaf(-cm, q[k][e], R[k][e]), 0.0f);
            j = j1;
          }
#pragma unroll
          for (int k = 0; k < kGroup; ++k) acc += (double)tree_sum(R[k]);
        }
      };
      bool full = false;  // (binary32 rows keep one form: with both, the pass spills registers)
      if constexpr (E::kBytes == 2) full = nvec == kVecPerLane * kWave;
      if (full) {
        if constexpr (E::kBytes == 2) pass(std::true_type{});
      } else {
        pass(std::false_type{});
      }
    } else {  // split on the target row's 16-byte grid: body vectors, then the lane's edge element
      const TreeSplit s = tree_split<E>(trow, V, c0, n);
      const int32_t e = split_edge(s, n, E::kPerVec, lane);
      constexpr int kGroup = kTreeGroup;
      for (int g0 = 0; g0 < kVecPerLane && g0 * kWave < s.body; g0 += kGroup) {
        float R[kGroup][E::kPerVec];
        int jc[kGroup];
#pragma unroll
        for (int k = 0; k < kGroup; ++k) {
          const int j = lane + kWave * (g0 + k);
          jc[k] = min(j, s.body - 1);
          float z[E::kPerVec];
          const u32x4 t = s.tv[jc[k]];
          E::unpack(j < s.body ? t : neg_inf_vec<E>(), z);
#pragma unroll
          for (int q = 0; q < E::kPerVec; ++q) R[k][q] = chain_p(f, z[q]);
        }
        for (int j = 0; j < f.l;) {
          const int j1 = chain_run_end(f, j);
          const char* dp = row_ptr<E>(draft, f.drow[j], V);
          uintptr_t pieces;
          uint32_t shift;
          split::tree_pieces(split::Plan{s.head, s.body, 0u, 0, 0}, (uintptr_t)dp, E::kBytes, c0, &pieces, &shift);
          const u32x4* dv = reinterpret_cast<const u32x4*>(at_address(dp, pieces));
          u32x4 b[kGroup];
          if (__builtin_amdgcn_readfirstlane(shift) == 0) {  // the draft row on the target's grid: one piece
#pragma unroll
            for (int k = 0; k < kGroup; ++k) b[k] = dv[jc[k]];
          } else {
#pragma unroll
            for (int k = 0; k < kGroup; ++k) b[k] = funnel16(dv[jc[k]], dv[jc[k] + 1], shift);
          }
          const float d_hi = f.d_hi[j];
          float q[kGroup][E::kPerVec];
#pragma unroll
          for (int k = 0; k < kGroup; ++k) {
            float z[E::kPerVec];
            E::unpack(b[k], z);
#pragma unroll
            for (int e2 = 0; e2 < E::kPerVec; ++e2) q[k][e2] = fast_exp2(fmaf(z[e2], f.k2, -d_hi));
          }
          const float c = run_mass(f, j, j1);
#pragma unroll
          for (int k = 0; k < kGroup; ++k)
#pragma unroll
            for (int e2 = 0; e2 < E::kPerVec; ++e2) R[k][e2] = fmaxf(fmaf(-c, q[k][e2], R[k][e2]), 0.0f);
          j = j1;
        }
#pragma unroll
        for (int k = 0; k < kGroup; ++k) acc += (double)tree_sum(R[k]);
      }
      if (e >= 0) acc += (double)chain_weight<E>(f, trow, draft, V, c0 + e);
    }
    acc = wave_sum(acc);
    if (lane == 0) lds_mass[c] = acc;
  }
}

// Inverse CDF inside one chunk by the whole workgroup: the chunk's vectors form 16 rows of 64
// (vector r*64 + l for lane l); wave w sums rows w, w + n_waves, ..., every wave scans the row sums,
// and the wave owning the crossing row recomputes its vectors, scans their sums across the lanes and
// walks the chosen vector.  A row off the 16-byte grid (kVec false) is split as tree_split says: two
// more segments, the head's elements before the rows and the tail's after them, weighed by wave 0
// and walked by it lane by lane.  kChain: the weights are R_l(v) of the frame f; else the node's own
// p in the frame 2^(z k - ref).  If rounding leaves the target unreached, the last element of
// positive weight is taken.  row_sums holds 18 doubles; the token is returned in every wave.
template <class E, bool kChain, bool kVec>
__device__ __forceinline__ int32_t tree_search_block(const ChainFrame& f, const char* trow, const void* draft,
                                                     int32_t V, int32_t c0, int32_t n, double target, float ref,
                                                     double* row_sums, int32_t* token, int lane, int wave,
                                                     int n_waves) {
  constexpr int kOff = kVec ? 0 : 1;            // off the grid the head's segment comes first
  constexpr int kSeg = kVecPerLane + 2 * kOff;  // the 16 rows (and the head and the tail)
  const int32_t nvec = n / E::kPerVec;
  TreeSplit s{0, nvec, reinterpret_cast<const u32x4*>(trow + (int64_t)c0 * E::kBytes)};
  if constexpr (!kVec) s = tree_split<E>(trow, V, c0, n);
  const int32_t b0 = c0 + s.head;  // the first body element
  auto weights = [&](int vi, float (&w)[E::kPerVec]) {
    float z[E::kPerVec];
    int jc = 0;
    if constexpr (kVec) {
      E::unpack(load_vec<E>(s.tv, vi, nvec), z);
    } else {
      jc = min(vi, s.body - 1);
      const u32x4 t = s.body > 0 ? s.tv[jc] : neg_inf_vec<E>();
      E::unpack(vi < s.body ? t : neg_inf_vec<E>(), z);
    }
    if constexpr (kChain) {
#pragma unroll
      for (int e = 0; e < E::kPerVec; ++e) w[e] = chain_p(f, z[e]);
      for (int j = 0; j < f.l;) {
        const int j1 = chain_run_end(f, j);
        const char* dp = row_ptr<E>(draft, f.drow[j], V);
        float zd[E::kPerVec];
        if constexpr (kVec)
          E::unpack(load_vec<E>(reinterpret_cast<const u32x4*>(dp + (int64_t)c0 * E::kBytes), vi, nvec), zd);
        else
          E::unpack(s.body > 0 ? tree_draft_vec<E>(dp, c0, s, jc) : neg_inf_vec<E>(), zd);
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e) w[e] = chain_run(f, j, j1, w[e], zd[e]);
        j = j1;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E::kPerVec; ++e) w[e] = fast_exp2(fmaf(z[e], f.k2, -ref));
    }
  };
  for (int r = wave; r < kVecPerLane; r += n_waves) {
    float w[E::kPerVec];
    weights(r * kWave + lane, w);
    const double rs = wave_sum((double)tree_sum(w));
    if (lane == 0) row_sums[kOff + r] = rs;
  }
  int32_t e = -1;
  float ew = 0.0f;
  if constexpr (!kVec) {
    e = split_edge(s, n, E::kPerVec, lane);
    if (wave == 0) {
      if (e >= 0)
        ew = kChain ? chain_weight<E>(f, trow, draft, V, c0 + e) : fast_exp2(fmaf(E::at(trow, c0 + e), f.k2, -ref));
      const double hs = wave_sum(lane < s.head ? (double)ew : 0.0);
      const double ts = wave_sum(lane < s.head ? 0.0 : (double)ew);
      if (lane == 0) {
        row_sums[0] = hs;
        row_sums[kSeg - 1] = ts;
      }
    }
  }
  __syncthreads();
  const double rsum = lane < kSeg ? row_sums[lane] : 0.0;
  const double rex = wave_exclusive_scan(rsum, lane);
  const uint64_t rhit = __ballot(lane < kSeg && rex + rsum > target);
  const uint64_t rpos = __ballot(lane < kSeg && rsum > 0.0);
  if (!rhit && !rpos) {
    if (wave == 0 && lane == 0) *token = c0 + n - 1;
  } else {
    const int kr = rhit ? __ffsll((unsigned long long)rhit) - 1 : 63 - __clzll((long long)rpos);
    const double rest = target - lane_value(rex, kr);
    if (!kVec && (kr == 0 || kr == kSeg - 1)) {  // an edge segment (positive sum): wave 0 walks its lanes
      if (wave == 0) {
        const bool mine = e >= 0 && (kr == 0) == (lane < s.head);
        const double w = mine ? (double)ew : 0.0;
        const double ex = wave_exclusive_scan(w, lane);
        const uint64_t hit = __ballot(rhit && mine && ex + w > rest);
        const uint64_t pos = __ballot(mine && w > 0.0);
        const int l = hit ? __ffsll((unsigned long long)hit) - 1 : 63 - __clzll((long long)pos);
        const int32_t y = lane_value(c0 + e, l);
        if (lane == 0) *token = y;
      }
    } else if (wave == (kr - kOff) % n_waves) {
      const int r = kr - kOff;
      float w[E::kPerVec];
      weights(r * kWave + lane, w);  // the same weights as the row sum's
      const float v = tree_sum(w);
      const double vex = wave_exclusive_scan((double)v, lane);
      const uint64_t vhit = __ballot(rhit && vex + (double)v > rest);
      const uint64_t vpos = __ballot(v > 0.0f);
      const int l = vhit ? __ffsll((unsigned long long)vhit) - 1 : (vpos ? 63 - __clzll((long long)vpos) : 63);
      const int32_t base = b0 + (r * kWave + lane) * E::kPerVec;
      int32_t yl = base + E::kPerVec - 1, last_pos = -1;
      double upto = vex;
      bool found = false;
#pragma unroll
      for (int q = 0; q < E::kPerVec; ++q) {
        upto += (double)w[q];
        if (w[q] > 0.0f) last_pos = base + q;
        if (!found && upto > rest) {
          yl = base + q;
          found = true;
        }
      }
      if (!vhit) yl = last_pos >= 0 ? last_pos : yl;
      const int32_t y = lane_value(yl, l);
      if (lane == 0) *token = y;
    }
  }
  __syncthreads();
  return *token;
}

// What wave 0 hands the workgroup after each step of the walk.
struct TreeStep {
  int32_t action;  // kTreePass: chunk masses of the frame's R_l; kTreeDraw: the extra token; kTreeDone
  int32_t kind;    // sdv_terminal_kind of the draw
  int32_t row;     // the current node's target row within the request (0: the root)
  int32_t token;   // T = 0: the extra token
  double u;        // T > 0: the draw's uniform
};
constexpr int32_t kTreePass = 0, kTreeDraw = 1, kTreeDone = 2;

template <class E, bool kGreedy, bool kVec>
__global__ __launch_bounds__(kWave * kTreeWaves) void tree_verdicts(Params P) {
  extern __shared__ double lds_mass[];  // [C], then staged records
  __shared__ RowFold rows[kMaxRows];
  __shared__ ChainFrame frame;
  __shared__ TreeStep step;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n_waves = blockDim.x / kWave;
  const int32_t i = blockIdx.x;
  const float k2 = P.k2;

  const int32_t lo_raw = P.cu[i], hi_raw = P.cu[i + 1];
  const bool ok_offsets = *P.batch_ok != 0;
  const int32_t lo = ok_offsets ? lo_raw : 0, hi = ok_offsets ? hi_raw : 0;
  const int N = hi - lo;
  const int32_t trow0 = lo + i, drow0 = lo;
  auto reject = [&](bool write_slots) {  // wave 0
    if (write_slots) {
      for (int j = lane; j <= N; j += kWave) P.out_tokens[trow0 + j] = -1;
      for (int j = lane; j < N; j += kWave) P.accepted_nodes[drow0 + j] = -1;
    }
    if (lane == 0) {
      P.accepted_len[i] = -1;
      if (P.dg.terminal_kind) P.dg.terminal_kind[i] = SDV_TERM_BAD;
    }
  };
  if (!ok_offsets || N > SDV_MAX_DEPTH) {  // malformed batch, or too many nodes: no slot written
    if (wave == 0) reject(false);
    return;
  }
  const float2* rec_t = P.part + (int64_t)trow0 * P.C;
  // the draft row of node j; an index outside the rows (the request is then rejected below) reads row 0
  auto draft_row_of = [&](int j) {
    const int32_t d = P.draft_row ? P.draft_row[drow0 + j] : drow0 + j;
    return (uint32_t)d < (uint32_t)P.n_dr ? d : 0;
  };
  auto draft_rec = [&](int j) { return P.part + (int64_t)(P.n_t + draft_row_of(j)) * P.C; };

  // 1. rows folded; wave 0 loads the nodes and, at T > 0, gathers z_t(x) from each node's parent row
  // and z_d(x) from its draft row
  const bool active = lane < N;
  int32_t x = 0, par = -1, qrow = 0;
  float zt = 0.0f, zd = 0.0f;
  bool bad_node = false;
  const int n_rows = kGreedy ? N + 1 : 2 * N + 1;
  stage_and_fold<kGreedy>(P, rec_t, draft_rec, N, n_rows, lds_mass, rows, lane, wave, n_waves, [&] {
    if (wave == 0 && active) {
      x = P.tokens[drow0 + lane];
      par = P.parents[drow0 + lane];
      const int32_t d = P.draft_row ? P.draft_row[drow0 + lane] : drow0 + lane;
      bad_node = x < 0 || x >= P.V || par < -1 || par >= lane || (!kGreedy && (d < 0 || d >= P.n_dr));
      qrow = bad_node ? 0 : d;
      if (!kGreedy && !bad_node) {
        zt = E::at(row_ptr<E>(P.target, trow0 + par + 1, P.V), x);
        zd = E::at(row_ptr<E>(P.draft, qrow, P.V), x);
      }
    }
  });

  // 2. the walk (wave 0), with a pass by the whole workgroup after each rejection.  Wave 0 keeps
  // the walk in registers: lane d the node accepted at depth d; lane j the draft row, its LSE and
  // M_j of the j-th rejected child of the current node.
  int a = 0;                   // accepted depth
  int32_t path_node = -1;      // lane d < a: the node accepted at depth d
  int32_t u = -1;              // the current node (-1: the root)
  int32_t cpos = 0;            // children of u below this node index have been tested
  int l = 0;                   // rejected children in the current residual
  bool rejected = false;       // some child of u was rejected
  double M_l = 1.0;            // mass of the current residual R_l
  int32_t rej_drow = 0;        // lane j < l: the rejected child's draft row
  double rej_l2 = 0.0, rej_m = 0.0;  // lane j < l: its draft row's base-2 LSE, and M_j
  double l2d_self = 0.0;       // lane n: the base-2 LSE of node n's draft row
  bool done = false;           // the request is rejected: nothing to draw
  if (wave == 0) {
    if (__ballot(active && bad_node) != 0 || (!kGreedy && __ballot(active && zd == -INFINITY) != 0)) {
      reject(true);  // a malformed node, or q(x) = 0 at some node: before any uniform is used
      done = true;
    } else if constexpr (!kGreedy) {
      if (active) l2d_self = rows[N + 1 + lane].l2;
      if (P.dg.target_lse)
        for (int r = lane; r <= N; r += kWave) P.dg.target_lse[trow0 + r] = rows[r].l2 * kLn2;
      if (active) {
        if (P.dg.draft_lse) P.dg.draft_lse[drow0 + lane] = l2d_self * kLn2;
        if (P.dg.target_logit) P.dg.target_logit[drow0 + lane] = zt;
        if (P.dg.draft_logit) P.dg.draft_logit[drow0 + lane] = zd;
      }
    }
  }
  for (;;) {
    if (wave == 0) {
      int32_t action = kTreeDone, token = -1;
      if (done) {
        // nothing: every wave leaves below
      } else if constexpr (kGreedy) {
        for (;;) {  // follow the first child equal to the node's argmax
          token = rows[u + 1].argmax;
          if (P.dg.target_argmax && lane == 0) P.dg.target_argmax[trow0 + u + 1] = token;
          const uint64_t hit = __ballot(active && par == u && x == token);
          if (!hit) break;
          const int32_t c = __ffsll((unsigned long long)hit) - 1;
          if (lane == a) path_node = c;
          ++a;
          u = c;
        }
        action = kTreeDraw;
      } else {
        for (;;) {
          const uint64_t kids = __ballot(active && par == u && lane >= cpos);
          if (!kids) {  // every child tested and rejected, or none: the extra token
            action = kTreeDraw;
            break;
          }
          const int32_t c = __ffsll((unsigned long long)kids) - 1;  // children in node order
          cpos = c + 1;
          const double l2u = rows[u + 1].l2, l2dc = lane_value(l2d_self, c);
          const double ztc = (double)lane_value(zt, c), zdc = (double)lane_value(zd, c);
          double ratio;
          if (l == 0) {  // the node's own p: log2 p(x)/q(x) = (z_t - z_d) k - (l2_t - l2_d)
            ratio = exp2((ztc - zdc) * (double)k2 - (l2u - l2dc));
          } else {  // R_l(x) / (M_l q(x)); lane j < l gathers rejected child j's draft logit at x
            const int32_t xc = lane_value(x, c);
            const float zj = lane < l ? E::at(row_ptr<E>(P.draft, rej_drow, P.V), xc) : 0.0f;
            double R = exp2(ztc * (double)k2 - l2u);
            for (int j = 0; j < l; ++j)
              R = fmax(R - lane_value(rej_m, j) * exp2((double)lane_value(zj, j) * (double)k2 - lane_value(rej_l2, j)),
                       0.0);
            ratio = R / (M_l * exp2(zdc * (double)k2 - l2dc));
          }
          const Philox4 blk = verifier_block(P.seed, (uint32_t)i, (uint32_t)c);
          const double r = (double)accept_uniform(blk);
          if (lane == 0) {
            if (P.dg.ratio) P.dg.ratio[drow0 + c] = ratio;
            if (P.dg.accept_uniform) P.dg.accept_uniform[drow0 + c] = (float)r;
          }
          if (r <= ratio) {  // accepted: c becomes the current node (its children follow it in node order)
            if (lane == a) path_node = c;
            ++a;
            u = c;
            l = 0;
            M_l = 1.0;
            rejected = false;
            continue;
          }
          // rejected: c joins the residual; the workgroup computes the chunk masses of R_{l+1}
          const int32_t qc = lane_value(qrow, c);
          if (lane == l) {
            rej_drow = qc;
            rej_l2 = l2dc;
            rej_m = M_l;
          }
          ++l;
          rejected = true;
          action = kTreePass;
          break;
        }
      }
      if (lane == 0) {
        step.action = action;
        step.row = u + 1;
        step.token = token;
        if constexpr (!kGreedy) {
          step.kind = !rejected ? SDV_TERM_BONUS : (l == 0 ? SDV_TERM_RESIDUAL_EMPTY : SDV_TERM_RESIDUAL);
          step.u = (double)draw_uniform(verifier_block(P.seed, (uint32_t)i, (uint32_t)(u + 1)));
        } else {
          step.kind = SDV_TERM_GREEDY;
        }
      }
      if constexpr (!kGreedy) {  // the residual's frame, for the pass and the in-chunk search
        if (!done) {
          const double l2 = rows[u + 1].l2;
          if (lane == 0) {
            frame.l = l;
            frame.k2 = k2;
            frame.t_hi = (float)l2;
            frame.t_lo = (float)(l2 - (double)(float)l2);
          }
          if (lane < l) {
            const double t_lo = (double)(float)(l2 - (double)(float)l2);
            const double d_lo = (double)(float)(rej_l2 - (double)(float)rej_l2);
            frame.drow[lane] = rej_drow;
            frame.d_hi[lane] = (float)rej_l2;
            frame.d_scale[lane] = (float)exp2(t_lo - d_lo);
            frame.m[lane] = (float)rej_m;
          }
        }
      }
    }
    __syncthreads();
    if (step.action != kTreePass) break;  // uniform: every wave read the same shared value
    chain_masses<E, kVec>(frame, row_ptr<E>(P.target, trow0 + step.row, P.V), P.draft, P.V, P.C, lds_mass, lane, wave,
                          n_waves);
    __syncthreads();
    if (wave == 0) {  // M_l; a residual without positive mass restarts from the node's own p
      double S = 0.0;
      for (int32_t c = lane; c < P.C; c += kWave) S += lds_mass[c];
      S = wave_sum(S) * exp2(-(double)frame.t_lo);  // from units of 2^-t_lo
      if (S > 0.0) {
        M_l = S;
      } else {
        l = 0;
        M_l = 1.0;
      }
    }
  }
  if (step.action != kTreeDraw) return;  // uniform: every wave read the same shared value

  // 3. the extra token (every wave picks the chunk, the whole workgroup searches it) and the outputs
  // (wave 0)
  const int32_t row = step.row;
  int32_t y = step.token;
  double S = 1.0;
  if constexpr (!kGreedy) {
    const char* tp = row_ptr<E>(P.target, trow0 + row, P.V);
    const bool chain = step.kind == SDV_TERM_RESIDUAL;  // R_l by the chunk masses of the last pass
    const float2* rec = rec_t + (int64_t)row * P.C;     // else the node's own p, by its records
    const float ref = rows[row].ref;                    // (the frame 2^(z k - ref))
    double tgt = 0.0;
    const int32_t cs =
        chain ? pick_chunk(P.C, step.u, [&](int32_t c) { return lds_mass[c]; }, &tgt, &S, lane)
              : pick_chunk(P.C, step.u, [&](int32_t c) { return (double)rec[c].y * exp2((double)rec[c].x - (double)ref); },
                           &tgt, &S, lane);
    const int32_t s0 = cs * E::kChunk, n = min(E::kChunk, P.V - s0);
    __shared__ int32_t drawn;
    y = chain ? tree_search_block<E, true, kVec>(frame, tp, P.draft, P.V, s0, n, tgt, ref, lds_mass + P.C, &drawn,
                                                 lane, wave, n_waves)
              : tree_search_block<E, false, kVec>(frame, tp, P.draft, P.V, s0, n, tgt, ref, lds_mass + P.C, &drawn,
                                                  lane, wave, n_waves);
    S *= chain ? exp2(-(double)frame.t_lo) : exp2((double)ref - rows[row].l2);  // probability units
  }
  if (wave != 0) return;
  const int32_t path_tok = __shfl(x, path_node < 0 ? 0 : path_node, kWave);
  for (int d = lane; d <= N; d += kWave) P.out_tokens[trow0 + d] = d < a ? path_tok : (d == a ? y : -1);
  for (int d = lane; d < N; d += kWave) P.accepted_nodes[drow0 + d] = d < a ? path_node : -1;
  if (lane == 0) {
    P.accepted_len[i] = a;
    if (P.dg.terminal_kind) P.dg.terminal_kind[i] = step.kind;
    if (!kGreedy && P.dg.draw_uniform) P.dg.draw_uniform[i] = (float)step.u;
    if (!kGreedy && P.dg.terminal_mass) P.dg.terminal_mass[i] = S;
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

// The verifier's blocks for requests i < B and positions j < P, laid out [i][j][4].
__global__ void philox_grid_kernel(uint64_t seed, int32_t B, int32_t P, uint32_t* __restrict__ words) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= (int64_t)B * P) return;
  const int32_t i = (int32_t)(b / P), j = (int32_t)(b - (int64_t)i * P);
  const Philox4 r = verifier_block(seed, (uint32_t)i, (uint32_t)j);
  words[4 * b] = r.w0;
  words[4 * b + 1] = r.w1;
  words[4 * b + 2] = r.w2;
  words[4 * b + 3] = r.w3;
}

// ============================================================================ read yardsticks
// Reads of whole 16 KiB chunks with no arithmetic, the words folded by xor so that no load is dead;
// each writes out[c] = the xor of chunk c's 4096 words.  Shape 0 is the row pass's (16-byte
// non-temporal register loads, one chunk per wave, four waves per workgroup): its rate is the
// bandwidth a one-pass stream of that shape reaches, the row pass's yardstick.  The other shapes
// check that yardstick against different ways of reading: direct-to-LDS loads in two-wave
// workgroups (1), and a persistent grid of eight workgroups per compute unit whose waves stride over
// the chunks with two in flight (2).

__device__ __forceinline__ uint32_t fold_chunk(const u32x4 (&buf)[kVecPerLane]) {
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < kVecPerLane; ++k) x ^= buf[k].x ^ buf[k].y ^ buf[k].z ^ buf[k].w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, kWave);
  return x;
}

constexpr int kLdsReadWaves = 2;
__global__ __launch_bounds__(kWave * kLdsReadWaves) void read_lds_kernel(const u32x4* __restrict__ src, int64_t n_chunks,
                                                                     uint32_t* __restrict__ out) {
  __shared__ u32x4 chunk_lds[kLdsReadWaves][kVecPerLane * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t c = (int64_t)blockIdx.x * kLdsReadWaves + wave;
  if (c >= n_chunks) return;
  u32x4 buf[kVecPerLane];
  load_chunk_lds<Bf16>(reinterpret_cast<const char*>(src + c * (kChunkBytes / 16)), 0, Bf16::kChunk, lane,
                       chunk_lds[wave], buf);
  const uint32_t x = fold_chunk(buf);
  if (lane == 0) out[c] = x;
}

__global__ __launch_bounds__(256) void read_reg_kernel(const u32x4* __restrict__ src, int64_t n_chunks,
                                                       uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t c = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (c >= n_chunks) return;
  const u32x4* v = src + c * (kChunkBytes / 16);
  u32x4 buf[kVecPerLane];
#pragma unroll
  for (int k = 0; k < kVecPerLane; ++k) buf[k] = __builtin_nontemporal_load(v + lane + kWave * k);
  const uint32_t x = fold_chunk(buf);
  if (lane == 0) out[c] = x;
}

__global__ __launch_bounds__(256) void read_strided_kernel(const u32x4* __restrict__ src, int64_t n_chunks,
                                                           uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t c = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave); c < n_chunks;
       c += 2 * waves) {
    const bool second = c + waves < n_chunks;
    const u32x4* v = src + c * (kChunkBytes / 16);
    const u32x4* w = src + (second ? c + waves : c) * (kChunkBytes / 16);
    u32x4 a[kVecPerLane], b[kVecPerLane];
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) a[k] = __builtin_nontemporal_load(v + lane + kWave * k);
#pragma unroll
    for (int k = 0; k < kVecPerLane; ++k) b[k] = __builtin_nontemporal_load(w + lane + kWave * k);
    const uint32_t xa = fold_chunk(a), xb = fold_chunk(b);
    if (lane == 0) {
      out[c] = xa;
      if (second) out[c + waves] = xb;
    }
  }
}

// ============================================================================ host side

struct Layout {
  int32_t C;
  int64_t n_t, slots;
  size_t part, cuts, hist, hist_top, pending, split_mass, split_count, total;  // hist, hist_top, pending: bf16 only
};

constexpr size_t kAlign = 256;
constexpr size_t kVerdictLdsBytes = 48 * 1024;  // dynamic shared memory of the verdict workgroup
constexpr int64_t kComputeUnits = 256;          // MI355X

// Verdict workgroups per request: a batch too small to occupy the compute units shares each
// correction's residual pass among several, four chunks apiece.  A compute unit's vector memory
// path bounds the pass, so spreading it over more units pays even with half of each workgroup's
// waves idle; below four chunks the publication of the masses costs more than the pass saves.
constexpr int32_t kSplitChunks = 4;
inline int32_t verdict_split(int32_t B, int32_t C) {
  const int64_t by_units = kComputeUnits / B, by_chunks = C / kSplitChunks;
  return (int32_t)std::max<int64_t>(1, std::min(by_units, by_chunks));
}
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Returns SDV_OK and fills the layout, or the status the shape violates.  counts: room for the
// key counts and the pending-row list of top-k / top-p calls on bf16 rows (calls that never
// truncate, such as sdv_verify, need none).
inline int make_layout(int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype, Layout* L, bool counts_room = true) {
  if (dtype != SDV_BF16 && dtype != SDV_FP32) return SDV_ERR_UNSUPPORTED;
  if (B < 1 || n_draft_rows < 0 || V < 1) return SDV_ERR_INVALID_ARG;
  const int64_t n_t = n_draft_rows + B;
  const int64_t slots = n_t + n_draft_rows;
  if (slots > INT32_MAX) return SDV_ERR_LIMIT;
  const int32_t chunk = dtype == SDV_BF16 ? Bf16::kChunk : F32::kChunk;
  const int32_t C = (int32_t)((V + (int64_t)chunk - 1) / chunk);
  if ((slots * C + 3) / 4 > INT32_MAX || C > kMaxChunks) return SDV_ERR_LIMIT;
  L->C = C;
  L->n_t = n_t;
  L->slots = slots;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L->part = take((size_t)slots * C * sizeof(float2));
  L->cuts = take((size_t)slots * sizeof(Cut));
  const bool bf16_counts = dtype == SDV_BF16 && counts_room;
  const size_t counts = bf16_counts ? (size_t)slots * C : 0;  // per-chunk key counts of truncating calls
  L->hist = take(counts * kHistKeys * sizeof(uint16_t));
  L->hist_top = take(counts * sizeof(uint32_t));
  L->pending = take(bf16_counts ? (size_t)(slots + 1) * sizeof(int32_t) : 0);
  L->split_mass = take((size_t)B * ((C + 15) / 16 * 16) * sizeof(double));
  L->split_count = take((size_t)B * kLineWords * sizeof(uint32_t) + sizeof(int32_t));  // counters, then the batch flag
  L->total = off;
  return SDV_OK;
}

inline dim3 row_grid(int64_t n_units, int waves) { return dim3((unsigned)((n_units + waves - 1) / waves)); }

// The row pass without counts, in workgroups of 8 waves when the stream is long enough (see kRowWaves).
template <class E, int kMode, bool kVec>
void launch_rows(const Params& P, hipStream_t stream) {
  if (kMode != kModeProfiled && P.n_units >= kWideRowUnits)
    hipLaunchKernelGGL((row_records<E, kMode, kVec, false, kWideRowWaves>), row_grid(P.n_units, kWideRowWaves),
                       dim3(kWave * kWideRowWaves), 0, stream, P);
  else
    hipLaunchKernelGGL((row_records<E, kMode, kVec, false>), row_grid(P.n_units, kRowWaves), dim3(kWave * kRowWaves), 0,
                       stream, P);
}

template <class E, int kMode, bool kVec>
int launch(Params& P, hipStream_t stream, const sdv_diag* diag) {
  auto record = [&](int k) {
    if (diag && diag->events[k]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(diag->events[k]), stream);
  };
  // the stream reads draft rows only when they are logits of a sampling rule
  P.n_units = (int64_t)(kMode == kModeGreedy || P.qrows ? P.n_t : P.n_t + P.n_d) * P.C;
  // top-k / top-p: the cut of every logit row the verdicts read (the greedy rule keeps its argmax
  // under any truncation, so it needs none); bf16 rows get per-chunk key counts from the row pass
  const bool cut = kMode != kModeGreedy && (P.top_k || P.top_p_milli);
  // verdict workgroups per request (the row pass zeroes their counters)
  P.split = kMode == kModeGreedy ? 1 : (P.split > 0 ? std::min(P.split, P.C) : verdict_split(P.B, P.C));
  // shared memory of the verdict workgroups: C residual masses, then as many chunk records as the
  // deepest request can need, up to the budget; deeper requests fold straight from the workspace
  const int64_t want = (int64_t)(2 * SDV_MAX_DEPTH + 1) * P.C;
  const int64_t room = (int64_t)(kVerdictLdsBytes - (size_t)P.C * sizeof(double)) / (int64_t)sizeof(float2);
  P.lds_records = want < room ? want : room;
  const size_t lds = (size_t)P.C * sizeof(double) + (size_t)P.lds_records * sizeof(float2);
  record(0);
  if constexpr (kMode != kModeProfiled && kVec) {  // (the split loads of rows off the 16-byte grid spill here)
    if (P.B == 1 && P.n_units <= kOneLaunchUnits && P.split == 1 && !cut && !P.qrows) {
      P.hist = nullptr;
      hipLaunchKernelGGL((one_launch<E, kMode>), dim3(1), dim3(kWave * kOneLaunchWaves), lds, stream, P);
      if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
      record(1);  // both passes ran in the one launch
      record(2);
      return SDV_OK;
    }
  }
  if constexpr (E::kBytes == 2 && kMode != kModeGreedy) {
    if (!cut) P.hist = nullptr;
    if (P.hist) {
      hipLaunchKernelGGL((row_records<E, kMode, kVec, true>), row_grid(P.n_units, kRowWaves), dim3(kWave * kRowWaves),
                         0, stream, P);
    } else {
      launch_rows<E, kMode, kVec>(P, stream);
    }
  } else {
    P.hist = nullptr;
    launch_rows<E, kMode, kVec>(P, stream);
  }
  if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
  record(1);
  if (cut) {
    const int64_t rows = P.qrows ? P.n_t : (int64_t)P.n_t + P.n_d;
    if (P.hist) {  // rows the counts settle; the rest are left pending for row_cuts
      hipLaunchKernelGGL((row_cuts_counted<kVec>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, P);
      if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
    }
    if constexpr (E::kBytes == 2) {
      if (P.hist) {  // the rows the count kernel left pending
        hipLaunchKernelGGL((row_cuts<E, kVec, true>), dim3((unsigned)rows), dim3(kCutThreads), 0, stream, P);
      } else {
        hipLaunchKernelGGL((row_cuts<E, kVec, false>), dim3((unsigned)rows), dim3(kCutThreads), 0, stream, P);
      }
    } else {
      hipLaunchKernelGGL((row_cuts<E, kVec, false>), dim3((unsigned)rows), dim3(kCutThreads), 0, stream, P);
    }
    if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
    record(3);
  }
  const dim3 grid((unsigned)P.B, (unsigned)P.split), block(kWave * kVerdictWaves);
  if constexpr (kMode != kModeGreedy) {  // the greedy rule never reads the draft side
    if (P.qrows) {
      if (cut) hipLaunchKernelGGL((verdicts<E, kMode, kVec, true, true>), grid, block, lds, stream, P);
      else hipLaunchKernelGGL((verdicts<E, kMode, kVec, true, false>), grid, block, lds, stream, P);
    } else if (cut) {
      hipLaunchKernelGGL((verdicts<E, kMode, kVec, false, true>), grid, block, lds, stream, P);
    } else {
      // a small batch of 16-byte rows of two to four chunks (the single pass over the whole pair):
      // 16 waves per request hide more of each correction's latency (64 x 32000 bf16: 11.8 against
      // 12.7 us of verdicts by rocprofv3); rows of one chunk (1 x 1000 fp32: 6.4 against 6.3 us),
      // long rows and full batches keep 8
      bool wide = false;
      if constexpr (kVec && kMode == kModeSampling)
        wide = P.split == 1 && P.C >= 2 && P.C <= 4 && 2 * (int64_t)P.B <= kComputeUnits;
      if (wide) {
        if constexpr (kVec && kMode == kModeSampling)
          hipLaunchKernelGGL((verdicts<E, kMode, kVec, false, false, kWideVerdictWaves>), grid,
                             dim3(kWave * kWideVerdictWaves), lds, stream, P);
      } else {
        hipLaunchKernelGGL((verdicts<E, kMode, kVec, false, false>), grid, block, lds, stream, P);
      }
    }
  } else {
    hipLaunchKernelGGL((verdicts<E, kMode, kVec, false, false>), grid, block, lds, stream, P);
  }
  if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
  record(2);
  return SDV_OK;
}

template <class E, int kMode>
int launch_vec(Params& P, bool vec, hipStream_t stream, const sdv_diag* diag) {
  return vec ? launch<E, kMode, true>(P, stream, diag) : launch<E, kMode, false>(P, stream, diag);
}

template <class E>
int launch_any(Params& P, bool vec, hipStream_t stream, const sdv_diag* diag) {
  if (P.temp_each) return launch_vec<E, kModeProfiled>(P, vec, stream, diag);
  if (P.k2 == 0.0f) return launch_vec<E, kModeGreedy>(P, vec, stream, diag);
  return launch_vec<E, kModeSampling>(P, vec, stream, diag);
}

// Token trees: the row pass as for linear drafts (the layout is the same), then one verdict
// workgroup per request walks its tree.
template <class E, bool kGreedy, bool kVec>
int launch_tree(Params& P, hipStream_t stream, const sdv_diag* diag) {
  auto record = [&](int k) {
    if (diag && diag->events[k]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(diag->events[k]), stream);
  };
  constexpr int kMode = kGreedy ? kModeGreedy : kModeSampling;
  P.n_units = (int64_t)(kGreedy ? P.n_t : P.n_t + P.n_dr) * P.C;
  P.hist = nullptr;
  P.split = 1;
  record(0);
  launch_rows<E, kMode, kVec>(P, stream);
  if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
  record(1);
  const int64_t want = (int64_t)(2 * SDV_MAX_DEPTH + 1) * P.C;
  const int64_t room = (int64_t)(kVerdictLdsBytes - (size_t)P.C * sizeof(double)) / (int64_t)sizeof(float2);
  P.lds_records = want < room ? want : room;
  const size_t lds = (size_t)P.C * sizeof(double) + (size_t)P.lds_records * sizeof(float2);
  hipLaunchKernelGGL((tree_verdicts<E, kGreedy, kVec>), dim3((unsigned)P.B), dim3(kWave * kTreeWaves), lds, stream, P);
  if (hipGetLastError() != hipSuccess) return SDV_ERR_HIP;
  record(2);
  return SDV_OK;
}

template <class E>
int launch_tree_any(Params& P, bool vec, hipStream_t stream, const sdv_diag* diag) {
  if (P.k2 == 0.0f)
    return vec ? launch_tree<E, true, true>(P, stream, diag) : launch_tree<E, true, false>(P, stream, diag);
  return vec ? launch_tree<E, false, true>(P, stream, diag) : launch_tree<E, false, false>(P, stream, diag);
}

// ---------------------------------------------------------------------------- the no-alloc entry point
// sdv_verify_noalloc keeps its workspace in this array instead of the caller's: each GPU the library
// runs on holds one copy, at its own address, until the process ends.  In host code the name stands
// for a host-side shadow, not a device address: kernels get the address hipGetSymbolAddress returns
// for the device that is current, looked up once per device and kept in noalloc_base.
static __device__ __align__(256) unsigned char scratch[SDV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex noalloc_mutex;
void* noalloc_base[kMaxDevices];  // the device address of scratch on each device, once looked up

// The address of the current device's copy of scratch, or null (with *status set) on failure.
void* noalloc_scratch(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    *status = SDV_ERR_HIP;
    return nullptr;
  }
  if (dev >= kMaxDevices) {
    *status = SDV_ERR_LIMIT;
    return nullptr;
  }
  std::lock_guard<std::mutex> hold(noalloc_mutex);
  if (!noalloc_base[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *status = SDV_ERR_HIP;
      return nullptr;
    }
    noalloc_base[dev] = ptr;
  }
  return noalloc_base[dev];
}

// Validation and launch shared by the entry points.  temp_each / seed_each are null for one profile
// per batch (temperature, seed), else device arrays of B values.
// Logits are read in their own width (and rows that are not 16-byte aligned in 16-byte pieces from
// the first 16-byte boundary on), so each base must sit on an element boundary.
bool element_aligned(const void* p, int32_t dtype) { return (uintptr_t)p % (dtype == SDV_BF16 ? 2 : 4) == 0; }

int verify_impl(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                double temperature, uint64_t seed, const sdv_options* opt, int32_t* accepted_len,
                int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream, const sdv_diag* diag,
                bool noalloc = false) {
  const bool counts_room = !noalloc;  // the static scratch holds no top-k / top-p counts
  const sdv_options none{};
  if (!opt) opt = &none;
  const float* temp_each = opt->temperature;
  const uint64_t* seed_each = opt->seed;
  if ((opt->accept_uniform == nullptr) != (opt->draw_uniform == nullptr)) return SDV_ERR_INVALID_ARG;
  if (opt->verdict_split < 0) return SDV_ERR_INVALID_ARG;
  if (opt->stop_offsets && (opt->n_stop_tokens < 0 || (opt->n_stop_tokens > 0 && !opt->stop_tokens)))
    return SDV_ERR_INVALID_ARG;
  Layout L;
  const int shape = make_layout(B, n_draft_rows, V, dtype, &L, counts_room);
  if (shape != SDV_OK) return shape;
  if (!counts_room && (opt->top_k || opt->top_p_milli)) return SDV_ERR_INVALID_ARG;
  if (!target_logits || !ragged_offsets || !accepted_len || !out_tokens) return SDV_ERR_INVALID_ARG;
  if (n_draft_rows > 0 && !draft_tokens) return SDV_ERR_INVALID_ARG;
  if (!element_aligned(target_logits, dtype) || !element_aligned(draft_logits, dtype) ||
      (uintptr_t)opt->draft_probs % 4 != 0)
    return SDV_ERR_INVALID_ARG;
  float k2 = 0.0f;  // 0 selects the greedy rule
  const bool profiled = temp_each != nullptr || seed_each != nullptr;
  const float* qrows = opt->draft_probs;
  const bool have_draft = draft_logits != nullptr || qrows != nullptr;
  if (profiled) {
    if (!temp_each || !seed_each || (n_draft_rows > 0 && !have_draft)) return SDV_ERR_INVALID_ARG;
  } else {
    if (!(temperature >= 0.0) || !isfinite(temperature)) return SDV_ERR_INVALID_ARG;
    if (temperature > 0.0) {
      k2 = (float)(1.4426950408889634074 / temperature);  // log2(e) / T
      if (!isfinite(k2) || !(k2 > 0.0f)) return SDV_ERR_INVALID_ARG;
      if (n_draft_rows > 0 && !have_draft) return SDV_ERR_INVALID_ARG;
    }
  }
  if (noalloc) {  // every argument has passed its checks: now the device's static scratch
    if (L.total > (size_t)SDV_NOALLOC_SCRATCH_BYTES) return SDV_ERR_LIMIT;
    int status = SDV_OK;
    workspace = noalloc_scratch(&status);
    if (!workspace) return status;
    workspace_bytes = SDV_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < L.total || (uintptr_t)workspace % kAlign != 0) return SDV_ERR_WORKSPACE;
  const int esize = dtype == SDV_BF16 ? 2 : 4;
  const void* draft = (profiled || k2 > 0.0f) && !qrows ? draft_logits : nullptr;
  const float* q = (profiled || k2 > 0.0f) ? qrows : nullptr;
  const bool vec = ((uintptr_t)target_logits % 16 == 0) && (draft == nullptr || (uintptr_t)draft % 16 == 0) &&
                   ((int64_t)V * esize) % 16 == 0 && (q == nullptr || ((uintptr_t)q % 16 == 0 && V % 4 == 0));
  char* ws = static_cast<char*>(workspace);
  Params P{};
  P.target = target_logits;
  P.draft = draft;
  P.tokens = draft_tokens;
  P.cu = ragged_offsets;
  P.accepted_len = accepted_len;
  P.out_tokens = out_tokens;
  P.part = reinterpret_cast<float2*>(ws + L.part);
  P.B = B;
  P.n_d = (int32_t)n_draft_rows;
  P.n_t = (int32_t)L.n_t;
  P.V = V;
  P.C = L.C;
  P.k2 = k2;
  P.seed = seed;
  P.temp_each = temp_each;
  P.seed_each = seed_each;
  P.r_each = opt->accept_uniform;
  P.u_each = opt->draw_uniform;
  P.stop_off = opt->stop_offsets;
  P.stop_tok = opt->stop_tokens;
  P.n_stop = opt->stop_offsets ? opt->n_stop_tokens : 0;
  P.budget = opt->budget;
  P.emitted_len = opt->emitted_len;
  P.qrows = q;
  P.top_k = opt->top_k;
  P.top_p_milli = opt->top_p_milli;
  P.kept_tokens = opt->kept_tokens;
  P.cuts = reinterpret_cast<Cut*>(ws + L.cuts);
  const bool bf16_counts = dtype == SDV_BF16 && counts_room;
  P.hist = bf16_counts ? reinterpret_cast<uint32_t*>(ws + L.hist) : nullptr;
  P.hist_top = bf16_counts ? reinterpret_cast<uint32_t*>(ws + L.hist_top) : nullptr;
  P.pending = bf16_counts ? reinterpret_cast<int32_t*>(ws + L.pending) : nullptr;
  P.split = opt->verdict_split;  // 0: chosen at launch
  P.split_mass = reinterpret_cast<double*>(ws + L.split_mass);
  P.split_count = reinterpret_cast<uint32_t*>(ws + L.split_count);
  P.batch_ok = reinterpret_cast<int32_t*>(P.split_count + (int64_t)B * kLineWords);
  P.Cm = (L.C + 15) / 16 * 16;
  if (diag) {
    P.dg = DiagPtrs{diag->target_lse,     diag->draft_lse,    diag->target_argmax, diag->ratio,
                    diag->accept_uniform, diag->draw_uniform, diag->terminal_kind, diag->target_logit,
                    diag->draft_logit,    diag->terminal_mass};
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == SDV_BF16) return launch_any<Bf16>(P, vec, s, diag);
  return launch_any<F32>(P, vec, s, diag);
}

int verify_tree_impl(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                     const int32_t* parents, const int32_t* draft_row, const int32_t* ragged_offsets, int32_t B,
                     int64_t n_nodes, int64_t n_draft_rows, int32_t V, int32_t dtype, double temperature,
                     uint64_t seed, int32_t* accepted_len, int32_t* accepted_nodes, int32_t* out_tokens,
                     void* workspace, size_t workspace_bytes, void* stream, const sdv_diag* diag) {
  Layout L;
  const int shape = make_layout(B, n_nodes, V, dtype, &L);
  if (shape != SDV_OK) return shape;
  if (!target_logits || !ragged_offsets || !accepted_len || !out_tokens) return SDV_ERR_INVALID_ARG;
  if (n_nodes > 0 && (!draft_tokens || !parents || !accepted_nodes)) return SDV_ERR_INVALID_ARG;
  if (!element_aligned(target_logits, dtype) || !element_aligned(draft_logits, dtype)) return SDV_ERR_INVALID_ARG;
  // draft rows: one per node, or (with indices) at most one per node, so the workspace holds them
  if (draft_row ? (n_draft_rows < 0 || n_draft_rows > n_nodes) : n_draft_rows != n_nodes) return SDV_ERR_INVALID_ARG;
  if (!(temperature >= 0.0) || !isfinite(temperature)) return SDV_ERR_INVALID_ARG;
  float k2 = 0.0f;
  if (temperature > 0.0) {
    k2 = (float)(1.4426950408889634074 / temperature);
    if (!isfinite(k2) || !(k2 > 0.0f)) return SDV_ERR_INVALID_ARG;
    if (n_draft_rows > 0 && !draft_logits) return SDV_ERR_INVALID_ARG;
  }
  if (!workspace || workspace_bytes < L.total || (uintptr_t)workspace % kAlign != 0) return SDV_ERR_WORKSPACE;
  const int esize = dtype == SDV_BF16 ? 2 : 4;
  const void* draft = k2 > 0.0f ? draft_logits : nullptr;
  const bool vec = ((uintptr_t)target_logits % 16 == 0) && (draft == nullptr || (uintptr_t)draft % 16 == 0) &&
                   ((int64_t)V * esize) % 16 == 0;
  char* ws = static_cast<char*>(workspace);
  Params P{};
  P.target = target_logits;
  P.draft = draft;
  P.tokens = draft_tokens;
  P.parents = parents;
  P.draft_row = draft_row;
  P.n_dr = (int32_t)n_draft_rows;
  P.accepted_nodes = accepted_nodes;
  P.cu = ragged_offsets;
  P.accepted_len = accepted_len;
  P.out_tokens = out_tokens;
  P.part = reinterpret_cast<float2*>(ws + L.part);
  P.B = B;
  P.n_d = (int32_t)n_nodes;
  P.n_t = (int32_t)L.n_t;
  P.V = V;
  P.C = L.C;
  P.k2 = k2;
  P.seed = seed;
  P.cuts = reinterpret_cast<Cut*>(ws + L.cuts);
  P.split_mass = reinterpret_cast<double*>(ws + L.split_mass);
  P.split_count = reinterpret_cast<uint32_t*>(ws + L.split_count);
  P.batch_ok = reinterpret_cast<int32_t*>(P.split_count + (int64_t)B * kLineWords);
  P.Cm = (L.C + 15) / 16 * 16;
  if (diag) {
    P.dg = DiagPtrs{diag->target_lse,     diag->draft_lse,    diag->target_argmax, diag->ratio,
                    diag->accept_uniform, diag->draw_uniform, diag->terminal_kind, diag->target_logit,
                    diag->draft_logit,    diag->terminal_mass};
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == SDV_BF16) return launch_tree_any<Bf16>(P, vec, s, diag);
  return launch_tree_any<F32>(P, vec, s, diag);
}

}  // namespace sdv

extern "C" {

int sdv_verify_tree(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                    const int32_t* parents, const int32_t* draft_row, const int32_t* ragged_offsets, int32_t B,
                    int64_t n_nodes, int64_t n_draft_rows, int32_t V, int32_t dtype, double temperature,
                    uint64_t seed, int32_t* accepted_len, int32_t* accepted_nodes, int32_t* out_tokens,
                    void* workspace, size_t workspace_bytes, void* stream, const sdv_diag* diag) {
  return sdv::verify_tree_impl(target_logits, draft_logits, draft_tokens, parents, draft_row, ragged_offsets, B,
                               n_nodes, n_draft_rows, V, dtype, temperature, seed, accepted_len, accepted_nodes,
                               out_tokens, workspace, workspace_bytes, stream, diag);
}

size_t sdv_noalloc_bytes(int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype) {
  sdv::Layout L;
  return sdv::make_layout(B, n_draft_rows, V, dtype, &L, false) == SDV_OK ? L.total : 0;
}

int sdv_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                       const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                       double temperature, uint64_t seed, int32_t* accepted_len, int32_t* out_tokens, void* stream) {
  return sdv::verify_impl(target_logits, draft_logits, draft_tokens, ragged_offsets, B, n_draft_rows, V, dtype,
                          temperature, seed, nullptr, accepted_len, out_tokens, nullptr, 0, stream, nullptr, true);
}


size_t sdv_workspace_bytes(int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype) {
  sdv::Layout L;
  return sdv::make_layout(B, n_draft_rows, V, dtype, &L) == SDV_OK ? L.total : 0;
}

int sdv_verify_ex(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                  const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                  double temperature, uint64_t seed, int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                  size_t workspace_bytes, void* stream, const sdv_diag* diag) {
  return sdv::verify_impl(target_logits, draft_logits, draft_tokens, ragged_offsets, B, n_draft_rows, V, dtype,
                          temperature, seed, nullptr, accepted_len, out_tokens, workspace, workspace_bytes, stream,
                          diag);
}

int sdv_verify_opts(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                    const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                    double temperature, uint64_t seed, const sdv_options* options, int32_t* accepted_len,
                    int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream,
                    const sdv_diag* diag) {
  return sdv::verify_impl(target_logits, draft_logits, draft_tokens, ragged_offsets, B, n_draft_rows, V, dtype,
                          temperature, seed, options, accepted_len, out_tokens, workspace, workspace_bytes, stream,
                          diag);
}

int sdv_verify_profiled(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                        const float* temperature, const uint64_t* seed, int32_t* accepted_len, int32_t* out_tokens,
                        void* workspace, size_t workspace_bytes, void* stream, const sdv_diag* diag) {
  if (!temperature || !seed) return SDV_ERR_INVALID_ARG;
  sdv_options opt{};
  opt.temperature = temperature;
  opt.seed = seed;
  return sdv::verify_impl(target_logits, draft_logits, draft_tokens, ragged_offsets, B, n_draft_rows, V, dtype, 0.0,
                          0, &opt, accepted_len, out_tokens, workspace, workspace_bytes, stream, diag);
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

int sdv_philox_uniforms(uint64_t seed, int32_t B, int32_t P, uint32_t* words, void* stream) {
  if (!words || B < 1 || P < 1) return SDV_ERR_INVALID_ARG;
  const int64_t n = (int64_t)B * P;
  if (n > INT32_MAX) return SDV_ERR_LIMIT;
  hipLaunchKernelGGL(sdv::philox_grid_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), seed, B, P, words);
  return hipGetLastError() == hipSuccess ? SDV_OK : SDV_ERR_HIP;
}

int sdv_read_yardstick(const void* src, int64_t n_chunks, int32_t shape, uint32_t* out, void* stream) {
  if (!src || !out || n_chunks < 1 || (uintptr_t)src % 16 != 0 || shape < 0 || shape > 2) return SDV_ERR_INVALID_ARG;
  if ((n_chunks + 1) / 2 > INT32_MAX) return SDV_ERR_LIMIT;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const sdv::u32x4* v = static_cast<const sdv::u32x4*>(src);
  if (shape == 0) {
    hipLaunchKernelGGL(sdv::read_reg_kernel, dim3((unsigned)((n_chunks + 3) / 4)), dim3(256), 0, s, v, n_chunks, out);
  } else if (shape == 1) {
    hipLaunchKernelGGL(sdv::read_lds_kernel,
                       dim3((unsigned)((n_chunks + sdv::kLdsReadWaves - 1) / sdv::kLdsReadWaves)),
                       dim3(sdv::kWave * sdv::kLdsReadWaves), 0, s, v, n_chunks, out);
  } else {
    const int64_t groups = std::min<int64_t>(8 * sdv::kComputeUnits, (n_chunks + 3) / 4);
    hipLaunchKernelGGL(sdv::read_strided_kernel, dim3((unsigned)groups), dim3(256), 0, s, v, n_chunks, out);
  }
  return hipGetLastError() == hipSuccess ? SDV_OK : SDV_ERR_HIP;
}

int sdv_read_ceiling(const void* src, int64_t n_chunks, uint32_t* out, void* stream) {
  return sdv_read_yardstick(src, n_chunks, 0, out, stream);
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
