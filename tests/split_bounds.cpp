// Walks the 16-byte split plans of csrc/split.hpp over many vocabularies, base offsets and rows, and
// checks on the host what the kernels rely on: the head, body and tail cover each chunk exactly,
// the edges fit one element per lane, every vector load is aligned and lies inside its chunk or
// row, and the second row's pieces put the right bytes under each vector.  Prints "ok <plans>".
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../lossless_draft_verification_online_amd/csrc/split.hpp"

using sdv::split::Plan;

static long g_plans = 0;

#define CHECK(cond, ...)                                                      \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::fprintf(stderr, "FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond);   \
      std::fprintf(stderr, __VA_ARGS__);                                      \
      std::fprintf(stderr, "\n");                                             \
      std::exit(1);                                                           \
    }                                                                         \
  } while (0)

// The edge lanes of a plan take each head and tail element exactly once.
static void check_edges(int32_t head, int32_t body_elems, int32_t n) {
  std::vector<int> seen(n > 0 ? n : 1, 0);
  for (int lane = 0; lane < 64; ++lane) {
    const int32_t e = sdv::split::edge(head, body_elems, n, lane);
    if (e < 0) continue;
    CHECK(e < n && (e < head || e >= head + body_elems), "edge %d head %d body %d n %d", e, head, body_elems, n);
    seen[e] += 1;
  }
  for (int32_t e = 0; e < n; ++e) {
    const bool is_edge = e < head || e >= head + body_elems;
    CHECK(seen[e] == (is_edge ? 1 : 0), "element %d seen %d (head %d body %d n %d)", e, seen[e], head, body_elems, n);
  }
}

// Vectors [first, first + 16 body) of a plan lie inside bytes [lo, hi) and are 16-byte aligned.
static void check_vectors(const Plan& p, uintptr_t lo, uintptr_t hi, const char* what) {
  if (p.body == 0) return;
  CHECK(p.first % 16 == 0, "%s: first %lx", what, (unsigned long)p.first);
  CHECK(p.first >= lo && p.first + 16 * (uintptr_t)p.body <= hi, "%s: vectors outside", what);
}

// Pieces of size kp under body units j in [0, body): piece j (and j + 1 when shift > 0) inside
// [r0, r1), aligned, and bytes pieces + kp j + shift are the row's bytes at element
// c0 + head + unit j.
static void check_pieces(uintptr_t pieces, uint32_t shift, int32_t body, uintptr_t kp, uintptr_t r0, uintptr_t r1,
                         uintptr_t want0, const char* what) {
  if (body == 0) return;
  CHECK(pieces % kp == 0 && shift < kp, "%s: pieces %lx shift %u", what, (unsigned long)pieces, shift);
  const uintptr_t last = pieces + kp * (uintptr_t)(body - 1) + (shift != 0 ? kp : 0);
  CHECK(pieces >= r0 && last + kp <= r1, "%s: pieces [%lx, %lx) outside row [%lx, %lx)", what, (unsigned long)pieces,
        (unsigned long)(last + kp), (unsigned long)r0, (unsigned long)r1);
  CHECK(pieces + shift == want0, "%s: bytes under unit 0 at %lx, want %lx", what, (unsigned long)(pieces + shift),
        (unsigned long)want0);
}

static void walk(int es, int32_t V, uintptr_t tbase, uintptr_t dbase, uintptr_t qbase, int row_t, int row_d) {
  const int P = 16 / es;
  const int32_t kChunk = 16384 / es;
  const uintptr_t tp = tbase + (uintptr_t)row_t * V * es, dp = dbase + (uintptr_t)row_d * V * es;
  const uintptr_t qp = qbase + (uintptr_t)row_d * V * 4;
  // the whole-row visitor: vectors from the first boundary, the tail after the last whole vector
  {
    const int32_t head = sdv::split::to_boundary(tp, es, V);
    const int32_t nvec = (V - head) / P, tail = V - head - nvec * P;
    CHECK(head >= 0 && head < P && tail >= 0 && tail < P, "visitor head %d tail %d V %d", head, tail, V);
    CHECK(nvec == 0 || (tp + (uintptr_t)head * es) % 16 == 0, "visitor vectors misaligned");
  }
  for (int32_t c0 = 0; c0 < V; c0 += kChunk) {
    const int32_t n = V - c0 < kChunk ? V - c0 : kChunk;
    const uintptr_t t0 = tp + (uintptr_t)c0 * es, t1 = t0 + (uintptr_t)n * es;
    // one row
    const Plan r = sdv::split::row(tp, es, c0, n);
    ++g_plans;
    CHECK(r.head >= 0 && r.body >= 0 && r.body <= 1024 && n - r.head - r.body * P >= 0, "row partition");
    CHECK(r.head < P || r.head == n, "row head %d", r.head);
    CHECK(n - r.head - r.body * P < P, "row tail");
    check_vectors(r, t0, t1, "row");
    CHECK(r.body == 0 || r.first == t0 + (uintptr_t)r.head * es, "row first");
    check_edges(r.head, r.body * P, n);
    // a row pair
    const Plan pp = sdv::split::pair(tp, dp, es, V, c0, n);
    ++g_plans;
    const int32_t ptail = n - pp.head - pp.body * P;
    CHECK(pp.head >= 0 && pp.body >= 0 && pp.body <= 1024 && ptail >= 0, "pair partition");
    CHECK(pp.head <= 2 * P - 1 && ptail <= 2 * P - 1, "pair edges %d %d", pp.head, ptail);
    check_vectors(pp, t0, t1, "pair target");
    CHECK(pp.body == 0 || pp.first == t0 + (uintptr_t)pp.head * es, "pair first");
    check_pieces(pp.pieces, pp.shift, pp.body, 16, dp, dp + (uintptr_t)V * es, dp + (uintptr_t)(c0 + pp.head) * es,
                 "pair draft");
    check_edges(pp.head, pp.body * P, n);
    // a tree node's row against draft rows at every element offset
    const Plan tr = sdv::split::tree(tp, es, V, c0, n);
    ++g_plans;
    const int32_t ttail = n - tr.head - tr.body * P;
    CHECK(tr.head >= 0 && tr.body >= 0 && tr.body <= 1024 && ttail >= 0, "tree partition");
    CHECK(tr.head <= 2 * P - 1 && ttail <= 2 * P - 1, "tree edges %d %d", tr.head, ttail);
    check_vectors(tr, t0, t1, "tree target");
    check_edges(tr.head, tr.body * P, n);
    for (int off = 0; off < P; ++off) {
      const uintptr_t d = dbase + (uintptr_t)off * es + (uintptr_t)(row_d + off) * V * es;
      uintptr_t pieces;
      uint32_t shift;
      sdv::split::tree_pieces(tr, d, es, c0, &pieces, &shift);
      check_pieces(pieces, shift, tr.body, 16, d, d + (uintptr_t)V * es, d + (uintptr_t)(c0 + tr.head) * es,
                   "tree draft");
    }
    // a (target row, q row) pair
    const Plan qq = sdv::split::q(tp, qp, es, V, c0, n);
    ++g_plans;
    const int32_t qtail = n - qq.head - qq.body * 4;
    CHECK(qq.head >= 0 && qq.body >= 0 && qq.body <= kChunk / 4 && qtail >= 0, "q partition");
    CHECK(qq.head <= 7 && qtail <= 7, "q edges %d %d", qq.head, qtail);
    const uintptr_t q0 = qp + (uintptr_t)c0 * 4;
    CHECK(qq.body == 0 || (qq.first % 16 == 0 && qq.first + 16 * (uintptr_t)qq.body <= q0 + (uintptr_t)n * 4 &&
                           qq.first == q0 + (uintptr_t)qq.head * 4),
          "q vectors");
    check_pieces(qq.pieces, qq.shift, qq.body, 4 * (uintptr_t)es, tp, tp + (uintptr_t)V * es,
                 tp + (uintptr_t)(c0 + qq.head) * es, "q target");
    check_edges(qq.head, qq.body * 4, n);
  }
}

int main() {
  std::vector<int32_t> vs;
  for (int32_t v = 1; v <= 300; ++v) vs.push_back(v);
  for (int32_t v : {511, 512, 513, 1000, 1001, 4095, 4096, 4097, 4099, 8191, 8192, 8193, 8195, 16383, 16384, 16385,
                    20011, 32000, 32003, 50257, 50264, 128255, 128256})
    vs.push_back(v);
  const uintptr_t kBase = (uintptr_t)1 << 32;  // addresses only: nothing is dereferenced
  for (int es : {2, 4}) {
    const int P = 16 / es;
    for (int32_t V : vs) {
      for (int toff = 0; toff < P; ++toff)
        for (int doff = 0; doff < P; doff += (V > 1000 ? 3 : 1))
          for (int qoff = 0; qoff < 4; qoff += (V > 1000 ? 3 : 1))
            for (int row = 0; row < (V > 1000 ? 3 : 5); ++row)
              walk(es, V, kBase + (uintptr_t)toff * es, 2 * kBase + (uintptr_t)doff * es, 3 * kBase + (uintptr_t)qoff * 4,
                   row, row + 1);
    }
  }
  std::printf("ok %ld\n", g_plans);
  return 0;
}
