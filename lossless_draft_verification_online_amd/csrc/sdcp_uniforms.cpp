// SDCP's verifier uniforms, computed on the host: HMAC-SHA-256 (RFC 2104 over FIPS 180-4 SHA-256)
// keyed with the sampling profile's seed ("Speculative Decoding Coordination Protocol (SDCP)",
// section "Acceptance Rules", Rule 2).  The values feed sdv_verify_opts as the caller's uniforms.
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "../../include/sdv.h"

namespace {

// ---------------------------------------------------------------- SHA-256 (FIPS 180-4, section 6.2)

constexpr uint32_t kRound[64] = {
    0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u, 0x3956c25bu, 0x59f111f1u, 0x923f82a4u, 0xab1c5ed5u,
    0xd807aa98u, 0x12835b01u, 0x243185beu, 0x550c7dc3u, 0x72be5d74u, 0x80deb1feu, 0x9bdc06a7u, 0xc19bf174u,
    0xe49b69c1u, 0xefbe4786u, 0x0fc19dc6u, 0x240ca1ccu, 0x2de92c6fu, 0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau,
    0x983e5152u, 0xa831c66du, 0xb00327c8u, 0xbf597fc7u, 0xc6e00bf3u, 0xd5a79147u, 0x06ca6351u, 0x14292967u,
    0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu, 0x53380d13u, 0x650a7354u, 0x766a0abbu, 0x81c2c92eu, 0x92722c85u,
    0xa2bfe8a1u, 0xa81a664bu, 0xc24b8b70u, 0xc76c51a3u, 0xd192e819u, 0xd6990624u, 0xf40e3585u, 0x106aa070u,
    0x19a4c116u, 0x1e376c08u, 0x2748774cu, 0x34b0bcb5u, 0x391c0cb3u, 0x4ed8aa4au, 0x5b9cca4fu, 0x682e6ff3u,
    0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u, 0x90befffau, 0xa4506cebu, 0xbef9a3f7u, 0xc67178f2u};

constexpr uint32_t kInit[8] = {0x6a09e667u, 0xbb67ae85u, 0x3c6ef372u, 0xa54ff53au,
                               0x510e527fu, 0x9b05688cu, 0x1f83d9abu, 0x5be0cd19u};

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

// One 64-byte block folded into the running hash state.
void compress(uint32_t h[8], const uint8_t block[64]) {
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t)block[4 * t] << 24 | (uint32_t)block[4 * t + 1] << 16 | (uint32_t)block[4 * t + 2] << 8 |
           (uint32_t)block[4 * t + 3];
  for (int t = 16; t < 64; ++t) {
    const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
    const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
    w[t] = w[t - 16] + s0 + w[t - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], k = h[7];
  for (int t = 0; t < 64; ++t) {
    const uint32_t t1 = k + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & f) ^ (~e & g)) + kRound[t] + w[t];
    const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) ^ (a & c) ^ (b & c));
    k = g;
    g = f;
    f = e;
    e = d + t1;
    d = c;
    c = b;
    b = a;
    a = t1 + t2;
  }
  h[0] += a;
  h[1] += b;
  h[2] += c;
  h[3] += d;
  h[4] += e;
  h[5] += f;
  h[6] += g;
  h[7] += k;
}

// SHA-256 of prefix (exactly one 64-byte block) followed by msg (len bytes): the message is padded
// with 0x80, zeros and its 64-bit bit length, big-endian.
void sha256_after_block(const uint8_t prefix[64], const uint8_t* msg, size_t len, uint8_t out[32]) {
  uint32_t h[8];
  memcpy(h, kInit, sizeof h);
  compress(h, prefix);
  uint8_t block[64];
  size_t off = 0;
  while (len - off >= 64) {
    compress(h, msg + off);
    off += 64;
  }
  const size_t rest = len - off;
  memset(block, 0, sizeof block);
  memcpy(block, msg + off, rest);
  block[rest] = 0x80;
  if (rest >= 56) {
    compress(h, block);
    memset(block, 0, sizeof block);
  }
  const uint64_t bits = (uint64_t)(64 + len) * 8;
  for (int b = 0; b < 8; ++b) block[56 + b] = (uint8_t)(bits >> (56 - 8 * b));
  compress(h, block);
  for (int q = 0; q < 8; ++q)
    for (int b = 0; b < 4; ++b) out[4 * q + b] = (uint8_t)(h[q] >> (24 - 8 * b));
}

// HMAC-SHA-256 (RFC 2104) with an 8-byte key: H((K ^ opad) || H((K ^ ipad) || m)), K zero-padded to
// the 64-byte block.
void hmac_sha256_key8(const uint8_t key[8], const uint8_t* msg, size_t len, uint8_t out[32]) {
  uint8_t ipad[64], opad[64], inner[32];
  memset(ipad, 0x36, sizeof ipad);
  memset(opad, 0x5c, sizeof opad);
  for (int b = 0; b < 8; ++b) {
    ipad[b] ^= key[b];
    opad[b] ^= key[b];
  }
  sha256_after_block(ipad, msg, len, inner);
  sha256_after_block(opad, inner, sizeof inner, out);
}

// One SDCP uniform: the first 53 bits of the HMAC, divided by 2^53, in [0, 1).
double sdcp_uniform(uint64_t seed, const uint8_t session[16], uint32_t round, uint32_t position, uint8_t purpose) {
  static const char kLabel[] = "SDCP-VERIFY-1";
  uint8_t key[8], msg[13 + 1 + 16 + 4 + 4 + 1];
  for (int b = 0; b < 8; ++b) key[b] = (uint8_t)(seed >> (56 - 8 * b));  // network byte order
  size_t n = 0;
  memcpy(msg, kLabel, 13);
  n += 13;
  msg[n++] = 0x00;
  memcpy(msg + n, session, 16);
  n += 16;
  for (int b = 0; b < 4; ++b) msg[n++] = (uint8_t)(round >> (24 - 8 * b));
  for (int b = 0; b < 4; ++b) msg[n++] = (uint8_t)(position >> (24 - 8 * b));
  msg[n++] = purpose;
  uint8_t mac[32];
  hmac_sha256_key8(key, msg, n, mac);
  uint64_t top = 0;
  for (int b = 0; b < 8; ++b) top = top << 8 | mac[b];
  return (double)(top >> 11) * 0x1.0p-53;
}

}  // namespace

extern "C" int sdv_sdcp_uniforms(int32_t B, const int32_t* cu, const uint64_t* seeds, const uint8_t* sessions,
                                 const uint32_t* rounds, double* accept_uniform, double* draw_uniform) {
  if (B < 1 || !cu || !seeds || !sessions || !rounds || !draw_uniform) return SDV_ERR_INVALID_ARG;
  if (cu[0] != 0) return SDV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < B; ++i)
    if (cu[i + 1] < cu[i] || cu[i + 1] - cu[i] > SDV_MAX_DEPTH) return SDV_ERR_INVALID_ARG;
  if (cu[B] > 0 && !accept_uniform) return SDV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < B; ++i) {
    const int32_t K = cu[i + 1] - cu[i];
    const uint8_t* session = sessions + 16 * (size_t)i;
    for (int32_t j = 0; j < K; ++j)  // acceptance tests at positions 1 .. K
      accept_uniform[cu[i] + j] = sdcp_uniform(seeds[i], session, rounds[i], (uint32_t)(j + 1), 0);
    for (int32_t t = 0; t <= K; ++t)  // the extra token drawn at position t + 1
      draw_uniform[(int64_t)cu[i] + i + t] = sdcp_uniform(seeds[i], session, rounds[i], (uint32_t)(t + 1), 1);
  }
  return SDV_OK;
}
