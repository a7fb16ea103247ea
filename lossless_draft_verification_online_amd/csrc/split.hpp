// Index arithmetic of the 16-byte splits that let rows off the 16-byte grid (an odd vocabulary, a
// base on an element boundary) be read with 16-byte vector loads.  Pure integer code on addresses,
// compiled for the device by the kernels and for the host by the bounds test, which walks every
// plan over many vocabularies, offsets and rows and checks that each load lies inside its row.
//
// A chunk [c0, c0 + n) of a row (element size es, 2 or 4 bytes, the row base on an element
// boundary) splits into head elements, `body` aligned 16-byte vectors and tail elements.  The head
// and tail are read one element per lane; the edge lane mapping is `edge`.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SDV_HD __host__ __device__ __attribute__((always_inline))  // a call in a kernel costs registers
#else
#define SDV_HD
#endif

namespace sdv {
namespace split {

struct Plan {
  int32_t head;    // elements before the first vector
  int32_t body;    // vectors (16 bytes of the first row each; 4 elements each for q plans)
  uint32_t shift;  // bytes from an aligned piece of the second row to the bytes under a vector
  uintptr_t first;   // address of vector 0 of the first row (16-byte aligned)
  uintptr_t pieces;  // address of the second row's piece 0 (aligned to the piece size)
};

SDV_HD inline int32_t min32(int32_t a, int32_t b) { return a < b ? a : b; }

// Elements from address a to the next 16-byte boundary, at most n.
SDV_HD inline int32_t to_boundary(uintptr_t a, int es, int32_t n) {
  return min32(n, (int32_t)((((a + 15) & ~(uintptr_t)15) - a) / (uintptr_t)es));
}

// One row: vectors from the first 16-byte boundary in the chunk on.
SDV_HD inline Plan row(uintptr_t rp, int es, int32_t c0, int32_t n) {
  Plan p;
  const uintptr_t b0 = rp + (uintptr_t)c0 * es;
  p.head = to_boundary(b0, es, n);
  p.body = (n - p.head) * es / 16;
  p.shift = 0;
  p.first = b0 + (uintptr_t)p.head * es;
  p.pieces = p.first;
  return p;
}

// A row pair on the first row's grid: the second row's bytes under vector j start `shift` bytes
// into its aligned vector pieces + 16 j and run into pieces + 16 (j + 1).  A vector whose pieces
// would reach outside the second row [dp, dp + V es) joins the head or the tail.
SDV_HD inline Plan pair(uintptr_t tp, uintptr_t dp, int es, int32_t V, int32_t c0, int32_t n) {
  Plan p = row(tp, es, c0, n);
  const uintptr_t x = dp + (uintptr_t)(c0 + p.head) * es;
  p.shift = (uint32_t)(x & 15);
  uintptr_t al = x - p.shift;
  if (p.body > 0 && al < dp) {  // the first low piece would start before the second row
    p.head += 16 / es;
    p.body -= 1;
    p.first += 16;
    al += 16;
  }
  const uintptr_t d_end = dp + (uintptr_t)V * es;
  if (p.body > 0 && p.shift != 0 && al + 16 * (uintptr_t)p.body + 16 > d_end) p.body -= 1;  // the last high piece
  p.pieces = al;
  return p;
}

// One target row against second rows at any offsets (token trees): while the first vector lies
// within 16 bytes of the row start it joins the head, and while the last ends within 16 bytes of
// the row end it joins the tail; then both pieces under any vector of any second row of V elements
// lie inside that row (tree_pieces gives them).
SDV_HD inline Plan tree(uintptr_t tp, int es, int32_t V, int32_t c0, int32_t n) {
  Plan p = row(tp, es, c0, n);
  if (p.body > 0 && (int64_t)(c0 + p.head) * es < 16) {
    p.head += 16 / es;
    p.body -= 1;
    p.first += 16;
  }
  if (p.body > 0 && (int64_t)(c0 + p.head) * es + 16 * (int64_t)p.body + 16 > (int64_t)V * es) p.body -= 1;
  return p;
}
SDV_HD inline void tree_pieces(const Plan& p, uintptr_t dp, int es, int32_t c0, uintptr_t* pieces, uint32_t* shift) {
  const uintptr_t x = dp + (uintptr_t)(c0 + p.head) * es;
  *shift = (uint32_t)(x & 15);
  *pieces = x - *shift;
}

// A (target row, q row) pair on the q row's grid (binary32 q, 4 values a vector): the 4 target
// logits under q vector j start `shift` bytes into the target's aligned pieces + kp j (kp = 4 es,
// 8 or 16 bytes) and run into the next piece.  A quad whose pieces would reach outside the target
// row joins the head or the tail.
SDV_HD inline Plan q(uintptr_t tp, uintptr_t qp, int es, int32_t V, int32_t c0, int32_t n) {
  const uintptr_t kp = 4 * (uintptr_t)es;
  Plan p;
  const uintptr_t q0 = qp + (uintptr_t)c0 * 4;
  p.head = to_boundary(q0, 4, n);
  p.body = (n - p.head) / 4;
  const uintptr_t x = tp + (uintptr_t)(c0 + p.head) * es;
  p.shift = (uint32_t)(x & (kp - 1));
  uintptr_t al = x - p.shift;
  if (p.body > 0 && al < tp) {  // the first low piece would start before the target row
    p.head += 4;
    p.body -= 1;
    al += kp;
  }
  const uintptr_t t_end = tp + (uintptr_t)V * es;
  if (p.body > 0 && p.shift != 0 && al + kp * (uintptr_t)p.body + kp > t_end) p.body -= 1;  // the last high piece
  p.first = qp + (uintptr_t)(c0 + p.head) * 4;
  p.pieces = al;
  return p;
}

// The chunk-relative element that lane `lane` takes at a plan's edges (lanes [0, head): the head,
// then the tail after the body's body_elems elements), or -1.
SDV_HD inline int32_t edge(int32_t head, int32_t body_elems, int32_t n, int lane) {
  const int32_t e = lane < head ? lane : head + body_elems + (lane - head);
  return e < n ? e : -1;
}

}  // namespace split
}  // namespace sdv
