/*
 * oracle/sdv_oracle.c -- fp64 CPU oracle for batched speculative-sampling verification.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline load this library.  The product path (the HIP library) never calls it, shares no
 * source with it, and must fail loudly rather than fall back to it.
 *
 * What it computes, and where the pages define it:
 *
 *  - Rule 1, greedy ("Speculative Decoding Coordination Protocol (SDCP)", section "Acceptance
 *    Rules", Rule 1; the temperature-zero tie rule is in section "Session Contract"): a draft
 *    token is accepted iff it equals the argmax of the target row, ties going to the smallest
 *    token id; evaluation stops at the first miss, and the extra token is the argmax of the row
 *    after the accepted prefix.
 *
 *  - Rule 2, speculative sampling (SDCP section "Acceptance Rules", Rule 2; "SOTA-227: Decode
 *    with a draft model and an accept-reject rule, which is exactly lossless", section "What to
 *    do", steps 3 and 4): walking the draft left to right, position j is accepted when
 *    r_j <= p_j(x_j) / q_j(x_j); at the first rejection the extra token is drawn from
 *    normalize(max(p_j - q_j, 0)); when every draft is accepted it is drawn from p at the
 *    position after the last draft.  A request with no drafts (K = 0) therefore draws one
 *    ordinary target token ("M7.8 - Speculative Serving", section 0x09, the K = 0 case).
 *
 *  - p and q are softmax(z / T) of the target and draft logit rows, then truncated by the
 *    request's top-k and top-p when it has them (SDCP "Session Contract": the sampling profile
 *    applies temperature, then top-k, then top-p, and p is the distribution after all three).
 *    The draft side gets the same profile, since the drafter samples from its own row under it.
 *
 *  - Token trees (multi-step speculative sampling over a tree of drafts, a published method the
 *    pages do not define): the section "token trees" below.
 *
 *  - Precondition (SDCP section "Verification and Commit", step 5): a proposal whose draft
 *    probability q_j(x_j) is zero at any position is rejected before any uniform is drawn.
 *    Out-of-range draft tokens and depths beyond 64 (SDCP "Session Contract", m_max <= 64) are
 *    rejected the same way.  A rejected request reports accepted_len = -1.
 *
 * Readings where the pages leave a step open:
 *  - uniforms: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *    1, 2, 3", SC'11) with key = (seed & 0xffffffff, seed >> 32) and counter =
 *    (position, request, 0, 0).  Word 0 feeds the accept test, word 1 the extra-token draw, which
 *    mirrors SDCP's two "purpose" values.  r = ((w0 >> 8) + 1) / 2^24 lies in (0, 1];
 *    u = (w1 >> 8) / 2^24 lies in [0, 1).  Both are exact in fp32 and fp64.
 *  - accept iff r <= ratio (the SOTA-227 form).  Since r > 0, a token with p(x) = 0 is never
 *    accepted, and ratio >= 1 always accepts.
 *  - the extra-token draw is the inverse CDF in ascending token id:
 *    y = min{ v : C(v) > u * S }, with C the inclusive prefix sum of the weights w and S = C(V-1).
 *    If rounding leaves no such v, y is the largest v with w_v > 0.
 *  - a residual with S = 0 (p == q exactly, which a rejection makes mathematically impossible)
 *    falls back to w = p.
 *  - top-k / top-p rank tokens by probability, equal probabilities (equal logits) going to the
 *    smaller token id, the one tie rule the pages state; top-k keeps the first top_k ranks (0, or
 *    top_k >= V, keeps all); top-p keeps the shortest run of leading ranks whose mass, renormalised
 *    over the top-k set, reaches top_p_milli / 1000, and never fewer than one token.  Given
 *    probability rows are used as they are (the drafter has applied its profile already).
 *
 * Everything is evaluated in fp64: bf16 and fp32 inputs convert to fp64 exactly, sums run in
 * ascending token order, and the residual is formed as p_v - q_v directly.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_DEPTH 64

enum { ORACLE_BF16 = 0, ORACLE_FP32 = 1 };

enum {
  ORACLE_TERM_GREEDY = 0,
  ORACLE_TERM_BONUS = 1,
  ORACLE_TERM_RESIDUAL = 2,
  ORACLE_TERM_RESIDUAL_EMPTY = 3,
  ORACLE_TERM_NONE = 4, /* stop token or budget within the accepted drafts: no extra token, no draw */
  ORACLE_TERM_BAD = -1
};

/* Optional per-row / per-position / per-request outputs.  Any pointer may be NULL. */
typedef struct {
  double* target_lse;     /* [n_target_rows]  LSE of z/T; written for every row of a valid request (T > 0) */
  double* draft_lse;      /* [n_draft_rows]   LSE of z/T; written for every row of a valid request (T > 0) */
  int32_t* target_argmax; /* [n_target_rows]  argmax, lowest index on ties (T == 0) */
  double* ratio;          /* [n_draft_rows]   p(x)/q(x) at every draft position of a valid request (T > 0) */
  double* accept_margin;  /* [n_draft_rows]   |r - ratio| at the positions actually tested, else NaN */
  double* cdf_margin;     /* [B]              margin of the extra-token draw, NaN when there was no draw */
  double* resid_mass;     /* [B]              S, the total weight of the extra-token draw */
  int32_t* terminal_kind; /* [B]              one of ORACLE_TERM_* */
  double* filter_margin;  /* [n_target_rows + n_draft_rows] relative distance of each truncated row's
                             top-p cut from its threshold; +inf where no top-p cut was taken */
} oracle_diag;

/*
 * Per-request options.  Every member may be NULL (0 for n_stop_tokens), which selects the
 * behaviour of oracle_verify.
 *  - temperature, seed [B]: one sampling profile per request (SDCP "Session Contract").
 *  - accept_uniform [n_draft_rows], draw_uniform [n_draft_rows + B]: uniforms in [0, 1) supplied
 *    by the caller, r per draft position and u per position (target-row layout).  With them the
 *    accept test is SDCP Rule 2's strict one, r < p/q.  Both or neither.
 *  - stop_offsets [B + 1], stop_tokens [n_stop_tokens]: request i stops at any of
 *    stop_tokens[stop_offsets[i] .. stop_offsets[i + 1]).
 *  - budget [B]: remaining output tokens of each request.
 *  - emitted_len [B] out: tokens emitted after truncation (SDCP "Verification and Commit", step 7;
 *    M7.8 section 0x09, "EOS and length-limit stopping").
 *  - draft_probs [n_draft_rows][V] binary32: the draft distributions themselves (SDCP's "q_rows",
 *    section "Message Definitions"), used as given in place of softmax(draft logits / T); the
 *    draft logits are then not read.  A zero (or negative, or NaN) q at a proposed token rejects
 *    the request before any draw (SDCP "Verification and Commit", step 5).
 *  - top_k [B], top_p_milli [B]: the rest of each request's sampling profile (SDCP "Session
 *    Contract": top_k a count, top_p_milli the nucleus mass in thousandths, at most 1000).
 *    top_k 0 and top_p_milli 1000 truncate nothing; a negative value, or top_p_milli above 1000,
 *    describes no profile and rejects the request.  Applied to p and to the draft logits' q at
 *    T > 0; a draft token outside q's kept set has q = 0 and rejects the request.
 *  - kept_tokens [n_draft_rows + B + n_draft_rows] out: tokens each row keeps after truncation,
 *    target rows first, then draft rows (V for a row that is not truncated); written for the
 *    rows of requests at T > 0 whose profile is valid.
 */
typedef struct {
  const double* temperature;
  const uint64_t* seed;
  const double* accept_uniform;
  const double* draw_uniform;
  const int32_t* stop_offsets;
  const int32_t* stop_tokens;
  int64_t n_stop_tokens;
  const int32_t* budget;
  int32_t* emitted_len;
  const float* draft_probs;
  const int32_t* top_k;
  const int32_t* top_p_milli;
  int32_t* kept_tokens;
} oracle_options;

/* ---------------------------------------------------------------- Philox4x32-10 (SC'11) */

/* One Philox4x32 round: two 32x32->64 products of the even counter words with the round
 * multipliers; the high halves are mixed with the odd words and the key, the low halves are
 * carried over, and the words are permuted. */
static void philox4x32_round(uint32_t x[4], const uint32_t k[2]) {
  const uint64_t prod_a = (uint64_t)0xD2511F53u * (uint64_t)x[0];
  const uint64_t prod_b = (uint64_t)0xCD9E8D57u * (uint64_t)x[2];
  const uint32_t y0 = (uint32_t)(prod_b >> 32) ^ x[1] ^ k[0];
  const uint32_t y1 = (uint32_t)prod_b;
  const uint32_t y2 = (uint32_t)(prod_a >> 32) ^ x[3] ^ k[1];
  const uint32_t y3 = (uint32_t)prod_a;
  x[0] = y0;
  x[1] = y1;
  x[2] = y2;
  x[3] = y3;
}

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { /* the key schedule adds the Weyl constants before every round but the first */
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox4x32_round(x, k);
  }
  memcpy(out, x, sizeof x);
}

/* The verifier's block for (request, position): key from the seed, counter (position, request, 0, 0). */
void oracle_philox_block(uint64_t seed, uint32_t request, uint32_t position, uint32_t out[4]) {
  const uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  const uint32_t ctr[4] = {position, request, 0u, 0u};
  oracle_philox4x32_10(ctr, key, out);
}

/* Blocks for requests 0..n_req-1 and positions 0..n_pos-1, laid out [request][position][4]. */
void oracle_philox_grid(uint64_t seed, int32_t n_req, int32_t n_pos, uint32_t* out) {
  for (int32_t i = 0; i < n_req; ++i)
    for (int32_t j = 0; j < n_pos; ++j)
      oracle_philox_block(seed, (uint32_t)i, (uint32_t)j, out + 4 * ((int64_t)i * n_pos + j));
}

/* r in (0, 1] for the accept test, from word 0. */
static double accept_uniform(const uint32_t w[4]) { return (double)((w[0] >> 8) + 1u) / 16777216.0; }
/* u in [0, 1) for the extra-token draw, from word 1. */
static double draw_uniform(const uint32_t w[4]) { return (double)(w[1] >> 8) / 16777216.0; }

/* ---------------------------------------------------------------- logit access */

static double logit_at(const void* base, int dtype, int64_t row, int32_t V, int32_t v) {
  const int64_t idx = row * (int64_t)V + v;
  if (dtype == ORACLE_BF16) {
    const uint16_t bits = ((const uint16_t*)base)[idx];
    uint32_t wide = (uint32_t)bits << 16; /* bf16 is the top half of an IEEE binary32 */
    float f;
    memcpy(&f, &wide, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

/* Natural-log LSE of z/T over one row: m/T + ln(sum_v exp((z_v - m)/T)), ascending v. */
double oracle_row_lse(const void* base, int dtype, int64_t row, int32_t V, double T) {
  double m = -INFINITY;
  for (int32_t v = 0; v < V; ++v) {
    const double z = logit_at(base, dtype, row, V, v);
    if (z > m) m = z;
  }
  if (m == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (int32_t v = 0; v < V; ++v) s += exp((logit_at(base, dtype, row, V, v) - m) / T);
  return m / T + log(s);
}

/* argmax over one row; the smallest index wins a tie (strict > while ascending). */
int32_t oracle_row_argmax(const void* base, int dtype, int64_t row, int32_t V) {
  int32_t best = 0;
  double best_z = logit_at(base, dtype, row, V, 0);
  for (int32_t v = 1; v < V; ++v) {
    const double z = logit_at(base, dtype, row, V, v);
    if (z > best_z) {
      best_z = z;
      best = v;
    }
  }
  return best;
}

/* ---------------------------------------------------------------- inverse-CDF draw */

/* y = min{v : C(v) > u*S}; returns y and its margin min(u - C(y-1)/S, C(y)/S - u). */
static int32_t inverse_cdf(const double* w, int32_t V, double u, double* S_out, double* margin) {
  double S = 0.0;
  for (int32_t v = 0; v < V; ++v) S += w[v];
  *S_out = S;
  const double target = u * S;
  double below = 0.0; /* C(v-1) */
  for (int32_t v = 0; v < V; ++v) {
    const double upto = below + w[v]; /* C(v) */
    if (upto > target) {
      const double lo = u - below / S, hi = upto / S - u;
      *margin = lo < hi ? lo : hi;
      return v;
    }
    below = upto;
  }
  /* rounding left u*S at or beyond C(V-1): the largest token with positive weight */
  for (int32_t v = V - 1; v >= 0; --v) {
    if (w[v] > 0.0) {
      *margin = 0.0;
      return v;
    }
  }
  *margin = 0.0;
  return V - 1;
}

/* ---------------------------------------------------------------- top-k / top-p */

/* A token as the sampling profile ranks it: the larger logit first (the larger probability), the
   smaller token id first among equal logits. */
typedef struct {
  double z;
  int32_t v;
} ranked_token;

static int rank_order(const void* pa, const void* pb) {
  const ranked_token* a = (const ranked_token*)pa;
  const ranked_token* b = (const ranked_token*)pb;
  if (a->z != b->z) return a->z > b->z ? -1 : 1;
  return a->v < b->v ? -1 : (a->v > b->v);
}

/* A profile that truncates nothing: top_k 0 (or at least V) and top_p_milli 1000. */
static int truncates(int64_t top_k, int32_t top_p_milli, int32_t V) {
  return (top_k > 0 && top_k < V) || top_p_milli < 1000;
}

/*
 * The tokens the sampling profile keeps in one row (SDCP "Session Contract": temperature, then
 * top-k, then top-p).  The row's tokens are sorted into rank order; top-k keeps the first top_k
 * ranks (all of them for 0 or top_k >= V); top-p then keeps the shortest run of leading ranks
 * whose mass exp((z - m) / T), divided by the mass of the top-k set, reaches top_p_milli / 1000,
 * and at least one token.
 *
 * keep [V] out: 1 for a kept token, 0 otherwise.  Returns the number of kept tokens and sets
 * *lse_kept = ln sum over kept v of exp(z_v / T), summed in ascending v, and *margin = the
 * distance of the top-p decision from its threshold relative to the top-k mass (+inf when top-p
 * takes no decision).  Returns -1 if scratch memory runs out.
 */
int32_t oracle_truncate_row(const void* base, int dtype, int64_t row, int32_t V, double T, int64_t top_k,
                            int32_t top_p_milli, unsigned char* keep, double* lse_kept, double* margin) {
  ranked_token* order = (ranked_token*)malloc(sizeof(ranked_token) * (size_t)V);
  if (!order) return -1;
  double m = -INFINITY;
  for (int32_t v = 0; v < V; ++v) {
    order[v].z = logit_at(base, dtype, row, V, v);
    order[v].v = v;
    if (order[v].z > m) m = order[v].z;
  }
  qsort(order, (size_t)V, sizeof *order, rank_order);
  int64_t n = (top_k > 0 && top_k < V) ? top_k : V;
  *margin = INFINITY;
  if (top_p_milli < 1000) {
    double mass_k = 0.0;
    for (int64_t r = 0; r < n; ++r) mass_k += exp((order[r].z - m) / T);
    const double target = mass_k * ((double)top_p_milli / 1000.0);
    double cum = 0.0;
    for (int64_t r = 0; r < n; ++r) {
      const double before = cum;
      cum += exp((order[r].z - m) / T);
      if (cum >= target) {
        /* the first rank is kept whatever its mass, so only later ranks have a lower side */
        const double over = (cum - target) / mass_k, under = (target - before) / mass_k;
        *margin = (r == 0 || over < under) ? over : under;
        n = r + 1;
        break;
      }
    }
  }
  memset(keep, 0, (size_t)V);
  for (int64_t r = 0; r < n; ++r) keep[order[r].v] = 1;
  free(order);
  double s = 0.0;
  for (int32_t v = 0; v < V; ++v)
    if (keep[v]) s += exp((logit_at(base, dtype, row, V, v) - m) / T);
  *lse_kept = m == -INFINITY ? -INFINITY : m / T + log(s);
  return (int32_t)n;
}

/* ---------------------------------------------------------------- one request */

static void set_nan(double* p) {
  if (p) *p = NAN;
}

/* Is token x one of request i's stop tokens? */
static int is_stop(const oracle_options* opt, int32_t i, int32_t x) {
  if (!opt || !opt->stop_offsets) return 0;
  for (int64_t s = opt->stop_offsets[i]; s < opt->stop_offsets[i + 1]; ++s)
    if (opt->stop_tokens[s] == x) return 1;
  return 0;
}

/*
 * How many of the a + 1 candidate tokens (a accepted drafts, then the extra token) are emitted:
 * none after the first stop token, and no more than the remaining budget.  The extra token is
 * emitted only when the count reaches a + 1 (SDCP "Verification and Commit", step 7; M7.8 section
 * 0x09: stopping inside the accepted drafts omits the correction or bonus).
 */
static int64_t emitted_count(const oracle_options* opt, int32_t i, const int32_t* drafts, int64_t a) {
  int64_t n = a + 1;
  for (int64_t j = 0; j < a; ++j)
    if (is_stop(opt, i, drafts[j])) {
      n = j + 1;
      break;
    }
  if (opt && opt->budget) {
    const int64_t b = opt->budget[i] > 0 ? opt->budget[i] : 0;
    if (b < n) n = b;
  }
  return n;
}

/* Is token v kept in row j of a request's truncated rows?  A NULL mask keeps every token. */
static int kept(const unsigned char* mask, int64_t j, int32_t V, int32_t v) {
  return !mask || mask[j * (int64_t)V + v];
}

/*
 * Request i.  n_t = n_draft_rows + B is the number of target rows (kept_tokens and filter_margin
 * hold the draft rows after them).  w: scratch of V doubles.
 */
static void verify_request(const void* target, const void* draft, int dtype, const int32_t* tokens,
                           const int32_t* cu, int32_t i, int64_t n_draft_rows, int64_t n_t, int32_t V, double T,
                           uint64_t seed, const oracle_options* opt, int32_t* accepted_len, int32_t* out_tokens,
                           oracle_diag* dg, double* w) {
  const int64_t lo = cu[i], hi = cu[i + 1];
  const int64_t K = hi - lo;
  int32_t* emitted = opt ? opt->emitted_len : NULL;
  if (emitted) emitted[i] = 0;
  if (dg && dg->cdf_margin) dg->cdf_margin[i] = NAN;
  if (dg && dg->resid_mass) dg->resid_mass[i] = NAN;
  if (lo < 0 || hi > n_draft_rows || K < 0 || K > ORACLE_MAX_DEPTH) {
    /* offsets that do not describe a valid request: no slot can be named, none is written */
    accepted_len[i] = -1;
    if (dg && dg->terminal_kind) dg->terminal_kind[i] = ORACLE_TERM_BAD;
    return;
  }
  const int64_t trow0 = lo + i; /* target rows of request i: trow0 .. trow0 + K */
  const int64_t drow0 = lo;     /* draft rows of request i:  drow0 .. drow0 + K - 1 */
  int32_t* slots = out_tokens + trow0;

  /* a temperature that is negative, NaN or infinite, a negative top_k, or a top_p_milli outside
     [0, 1000] describes no sampling profile; a stop list that does not lie inside the stop-token
     array describes no stop set */
  const int64_t top_k = opt && opt->top_k ? opt->top_k[i] : 0;
  const int32_t top_p_milli = opt && opt->top_p_milli ? opt->top_p_milli[i] : 1000;
  int bad = !(T >= 0.0) || isinf(T) || top_k < 0 || top_p_milli < 0 || top_p_milli > 1000;
  if (opt && opt->stop_offsets) {
    const int64_t s0 = opt->stop_offsets[i], s1 = opt->stop_offsets[i + 1];
    if (s0 < 0 || s1 < s0 || s1 > opt->n_stop_tokens) bad = 1;
  }
  for (int64_t j = 0; j < K && !bad; ++j)
    if (tokens[drow0 + j] < 0 || tokens[drow0 + j] >= V) bad = 1;

  /* Rule 2's rows: LSE of z/T over each row, or over its kept tokens when the profile truncates
     (the greedy rule needs neither: the argmax is always kept) */
  const float* qrows = opt ? opt->draft_probs : NULL;
  unsigned char* keep_t = NULL; /* [(K + 1) V] kept tokens of the target rows, NULL: all */
  unsigned char* keep_d = NULL; /* [K V] of the draft rows */
  double lse_t[ORACLE_MAX_DEPTH + 1], lse_d[ORACLE_MAX_DEPTH];
  if (!bad && T > 0.0) {
    const int cut = truncates(top_k, top_p_milli, V);
    if (cut) {
      keep_t = (unsigned char*)malloc((size_t)(K + 1) * (size_t)V);
      if (!qrows && K > 0) keep_d = (unsigned char*)malloc((size_t)K * (size_t)V);
      if (!keep_t || (!qrows && K > 0 && !keep_d)) abort(); /* test infrastructure: no partial answer */
    }
    for (int64_t j = 0; j <= K; ++j) {
      double margin = INFINITY;
      int32_t n = V;
      if (cut)
        n = oracle_truncate_row(target, dtype, trow0 + j, V, T, top_k, top_p_milli, keep_t + j * (int64_t)V,
                                &lse_t[j], &margin);
      else
        lse_t[j] = oracle_row_lse(target, dtype, trow0 + j, V, T);
      if (n < 0) abort();
      if (opt && opt->kept_tokens) opt->kept_tokens[trow0 + j] = n;
      if (dg && dg->filter_margin) dg->filter_margin[trow0 + j] = margin;
    }
    for (int64_t j = 0; j < K; ++j) {
      double margin = INFINITY;
      int32_t n = V;
      if (qrows) {
        lse_d[j] = NAN;
        continue;
      }
      if (cut)
        n = oracle_truncate_row(draft, dtype, drow0 + j, V, T, top_k, top_p_milli, keep_d + j * (int64_t)V,
                                &lse_d[j], &margin);
      else
        lse_d[j] = oracle_row_lse(draft, dtype, drow0 + j, V, T);
      if (n < 0) abort();
      if (opt && opt->kept_tokens) opt->kept_tokens[n_t + drow0 + j] = n;
      if (dg && dg->filter_margin) dg->filter_margin[n_t + drow0 + j] = margin;
    }
    /* q_j(x_j) = 0 when the draft logit at x_j is -inf, when x_j is outside the kept tokens of the
       draft row, or when the given probability at x_j is not positive; checked before any draw */
    for (int64_t j = 0; j < K; ++j) {
      const int32_t x = tokens[drow0 + j];
      if (qrows) {
        if (!(qrows[(drow0 + j) * (int64_t)V + x] > 0.0f)) bad = 1;
      } else if (logit_at(draft, dtype, drow0 + j, V, x) == -INFINITY || !kept(keep_d, j, V, x)) {
        bad = 1;
      }
    }
  }
  if (bad) {
    accepted_len[i] = -1;
    for (int64_t j = 0; j <= K; ++j) slots[j] = -1;
    if (dg && dg->terminal_kind) dg->terminal_kind[i] = ORACLE_TERM_BAD;
    free(keep_t);
    free(keep_d);
    return;
  }

  if (T == 0.0) { /* ---- Rule 1 */
    int64_t a = K;
    for (int64_t j = 0; j < K; ++j) {
      if (tokens[drow0 + j] != oracle_row_argmax(target, dtype, trow0 + j, V)) {
        a = j;
        break;
      }
    }
    if (dg && dg->target_argmax)
      for (int64_t j = 0; j <= K; ++j) dg->target_argmax[trow0 + j] = oracle_row_argmax(target, dtype, trow0 + j, V);
    const int64_t n = emitted_count(opt, i, tokens + drow0, a);
    for (int64_t j = 0; j <= K; ++j) slots[j] = -1;
    for (int64_t j = 0; j < a && j < n; ++j) slots[j] = tokens[drow0 + j];
    if (n == a + 1) slots[a] = oracle_row_argmax(target, dtype, trow0 + a, V);
    accepted_len[i] = (int32_t)a;
    if (emitted) emitted[i] = (int32_t)n;
    if (dg && dg->terminal_kind) dg->terminal_kind[i] = n == a + 1 ? ORACLE_TERM_GREEDY : ORACLE_TERM_NONE;
    return;
  }

  /* ---- Rule 2 */
  if (dg) {
    for (int64_t j = 0; j <= K; ++j)
      if (dg->target_lse) dg->target_lse[trow0 + j] = lse_t[j];
    for (int64_t j = 0; j < K; ++j) {
      if (dg->draft_lse && !qrows) dg->draft_lse[drow0 + j] = lse_d[j];
      set_nan(dg->accept_margin ? &dg->accept_margin[drow0 + j] : NULL);
    }
  }

  int64_t a = K;
  for (int64_t j = 0; j < K; ++j) {
    const int32_t x = tokens[drow0 + j];
    double ratio; /* p_j(x) / q_j(x); p_j(x) = 0 for a token the target row does not keep */
    if (!kept(keep_t, j, V, x)) {
      ratio = 0.0;
    } else if (qrows) {
      ratio = exp(logit_at(target, dtype, trow0 + j, V, x) / T - lse_t[j]) / (double)qrows[(drow0 + j) * (int64_t)V + x];
    } else {
      const double log_ratio =
          (logit_at(target, dtype, trow0 + j, V, x) - logit_at(draft, dtype, drow0 + j, V, x)) / T - (lse_t[j] - lse_d[j]);
      ratio = exp(log_ratio);
    }
    if (dg && dg->ratio) dg->ratio[drow0 + j] = ratio;
    if (a < K) continue; /* positions after the first rejection are never tested */
    int accept;
    double r;
    if (opt && opt->accept_uniform) { /* the caller's r in [0, 1): SDCP Rule 2, r < p/q */
      r = opt->accept_uniform[drow0 + j];
      accept = r < ratio;
    } else { /* Philox r in (0, 1]: r <= p/q */
      uint32_t blk[4];
      oracle_philox_block(seed, (uint32_t)i, (uint32_t)j, blk);
      r = accept_uniform(blk);
      accept = r <= ratio;
    }
    if (dg && dg->accept_margin) dg->accept_margin[drow0 + j] = fabs(r - ratio);
    if (!accept) a = j;
  }

  const int64_t t = a; /* the position whose extra token is drawn */
  const int64_t n_emit = emitted_count(opt, i, tokens + drow0, a);
  accepted_len[i] = (int32_t)a;
  if (emitted) emitted[i] = (int32_t)n_emit;
  if (n_emit < a + 1) { /* emission stops inside the accepted drafts: no extra token is drawn */
    for (int64_t j = 0; j <= K; ++j) slots[j] = j < n_emit ? tokens[drow0 + j] : -1;
    if (dg && dg->terminal_kind) dg->terminal_kind[i] = ORACLE_TERM_NONE;
    free(keep_t);
    free(keep_d);
    return;
  }
  double u;
  if (opt && opt->draw_uniform) {
    u = opt->draw_uniform[trow0 + t];
  } else {
    uint32_t blk[4];
    oracle_philox_block(seed, (uint32_t)i, (uint32_t)t, blk);
    u = draw_uniform(blk);
  }
  int kind;
  if (t < K) {
    kind = ORACLE_TERM_RESIDUAL;
    double S = 0.0;
    for (int32_t v = 0; v < V; ++v) {
      const double p = kept(keep_t, t, V, v) ? exp(logit_at(target, dtype, trow0 + t, V, v) / T - lse_t[t]) : 0.0;
      const double q = qrows ? (double)qrows[(drow0 + t) * (int64_t)V + v]
                             : (kept(keep_d, t, V, v) ? exp(logit_at(draft, dtype, drow0 + t, V, v) / T - lse_d[t]) : 0.0);
      w[v] = p > q ? p - q : 0.0;
      S += w[v];
    }
    if (!(S > 0.0)) {
      kind = ORACLE_TERM_RESIDUAL_EMPTY;
      for (int32_t v = 0; v < V; ++v)
        w[v] = kept(keep_t, t, V, v) ? exp(logit_at(target, dtype, trow0 + t, V, v) / T - lse_t[t]) : 0.0;
    }
  } else {
    kind = ORACLE_TERM_BONUS;
    for (int32_t v = 0; v < V; ++v)
      w[v] = kept(keep_t, t, V, v) ? exp(logit_at(target, dtype, trow0 + t, V, v) / T - lse_t[t]) : 0.0;
  }
  double S, margin;
  const int32_t y = inverse_cdf(w, V, u, &S, &margin);

  for (int64_t j = 0; j < t; ++j) slots[j] = tokens[drow0 + j];
  slots[t] = y;
  for (int64_t j = t + 1; j <= K; ++j) slots[j] = -1;
  if (dg) {
    if (dg->cdf_margin) dg->cdf_margin[i] = margin;
    if (dg->resid_mass) dg->resid_mass[i] = S;
    if (dg->terminal_kind) dg->terminal_kind[i] = kind;
  }
  free(keep_t);
  free(keep_d);
}

/* ---------------------------------------------------------------- batch entry point */

/*
 * target        [n_draft_rows + B][V]  row-major, dtype (0 = bf16 bits as uint16, 1 = fp32)
 * draft         [n_draft_rows][V]      may be NULL when T == 0
 * draft_tokens  [n_draft_rows]
 * cu            [B + 1] exclusive prefix sums of the per-request depths K_i
 * accepted_len  [B]     out
 * out_tokens    [n_draft_rows + B]  out: request i owns slots cu[i]+i .. cu[i]+i+K_i
 * Returns 0, or -1 for arguments that describe no batch.
 */
static int verify_batch(const void* target, const void* draft, int dtype, const int32_t* draft_tokens,
                        const int32_t* cu, int32_t B, int64_t n_draft_rows, int32_t V, double T, uint64_t seed,
                        const oracle_options* opt, int32_t* accepted_len, int32_t* out_tokens, oracle_diag* diag) {
  const double* T_each = opt ? opt->temperature : NULL;
  const uint64_t* seed_each = opt ? opt->seed : NULL;
  int failed = 0;
#pragma omp parallel reduction(| : failed)
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    if (!w) failed = 1;
#pragma omp for schedule(dynamic, 1)
    for (int32_t i = 0; i < B; ++i)
      if (w)
        verify_request(target, draft, dtype, draft_tokens, cu, i, n_draft_rows, n_draft_rows + B, V,
                       T_each ? T_each[i] : T,
                       seed_each ? seed_each[i] : seed, opt, accepted_len, out_tokens, diag, w);
    free(w);
  }
  return failed ? -2 : 0;
}

int oracle_verify(const void* target, const void* draft, int dtype, const int32_t* draft_tokens, const int32_t* cu,
                  int32_t B, int64_t n_draft_rows, int32_t V, double T, uint64_t seed, int32_t* accepted_len,
                  int32_t* out_tokens, oracle_diag* diag) {
  if (!target || !draft_tokens || !cu || !accepted_len || !out_tokens) return -1;
  if (B <= 0 || V <= 0 || n_draft_rows < 0 || !(T >= 0.0) || isinf(T) || (T > 0.0 && !draft)) return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP32) return -1;
  return verify_batch(target, draft, dtype, draft_tokens, cu, B, n_draft_rows, V, T, seed, NULL, accepted_len,
                      out_tokens, diag);
}

/*
 * The general entry point: T and seed as in oracle_verify, refined by the per-request options
 * (which may be NULL).  Per-request temperatures need draft logits whenever n_draft_rows > 0.
 */
int oracle_verify_opts(const void* target, const void* draft, int dtype, const int32_t* draft_tokens,
                       const int32_t* cu, int32_t B, int64_t n_draft_rows, int32_t V, double T, uint64_t seed,
                       const oracle_options* opt, int32_t* accepted_len, int32_t* out_tokens, oracle_diag* diag) {
  if (!target || !draft_tokens || !cu || !accepted_len || !out_tokens) return -1;
  if (B <= 0 || V <= 0 || n_draft_rows < 0) return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP32) return -1;
  const int profiled = opt && opt->temperature;
  if (opt && (!opt->temperature) != (!opt->seed)) return -1;
  if (opt && (!opt->accept_uniform) != (!opt->draw_uniform)) return -1;
  if (opt && opt->stop_offsets && (opt->n_stop_tokens < 0 || (opt->n_stop_tokens > 0 && !opt->stop_tokens))) return -1;
  const int have_draft = draft || (opt && opt->draft_probs);
  if (!profiled && (!(T >= 0.0) || isinf(T) || (T > 0.0 && !have_draft && n_draft_rows > 0))) return -1;
  if (profiled && n_draft_rows > 0 && !have_draft) return -1;
  return verify_batch(target, draft, dtype, draft_tokens, cu, B, n_draft_rows, V, T, seed, opt, accepted_len,
                      out_tokens, diag);
}

/*
 * The same with a sampling profile per request (SDCP "Session Contract": every session carries its
 * own profile, and a verification batch gathers many sessions).  temperature[i] and seed[i] apply
 * to request i: temperature 0 selects Rule 1 for that request, a positive one Rule 2; a negative,
 * NaN or infinite temperature rejects the request (accepted_len -1, all of its slots -1).  draft
 * may be NULL only when n_draft_rows == 0.
 */
int oracle_verify_profiled(const void* target, const void* draft, int dtype, const int32_t* draft_tokens,
                           const int32_t* cu, int32_t B, int64_t n_draft_rows, int32_t V, const double* temperature,
                           const uint64_t* seed, int32_t* accepted_len, int32_t* out_tokens, oracle_diag* diag) {
  if (!temperature || !seed) return -1;
  oracle_options opt = {temperature, seed, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL};
  return oracle_verify_opts(target, draft, dtype, draft_tokens, cu, B, n_draft_rows, V, 0.0, 0, &opt, accepted_len,
                            out_tokens, diag);
}

/* ---------------------------------------------------------------- token trees
 *
 * Tree verification by multi-step speculative sampling: Miao et al., "SpecInfer: Accelerating
 * Large Language Model Serving with Tree-based Speculative Inference and Verification" (ASPLOS
 * 2024), section 4, the token tree verifier and its stochastic rule.  The pages define no tree rule
 * (SDCP section "Scope" leaves tree-structured speculation out of its first version; M7.8 names
 * trees among the proposal shapes a verifier meets); this is the reading taken:
 *
 *  - request i has N_i nodes n = 0 .. N_i - 1 (offsets cu as for linear drafts, N_i <= 64); node
 *    n has parent parents[cu[i] + n] in [-1, n - 1] (-1: the root, the last committed token) and
 *    token tokens[cu[i] + n], sampled from q_n = softmax(draft row d / T), the drafter's
 *    distribution at its parent's context, with d = draft_row[cu[i] + n] when the caller gives
 *    row indices (siblings from one drafter then share one row) and d = cu[i] + n otherwise;
 *  - target rows: cu[i] + i at the root, cu[i] + i + n + 1 after node n; a chain (node n the
 *    parent of node n + 1) is exactly a linear draft;
 *  - Rule 2 (T > 0): at the current node, with p its target distribution, the children are tested
 *    in ascending node order.  Child c is accepted iff r_c <= p(x_c) / q_c(x_c), and the walk moves
 *    to c with p = c's target distribution.  On a rejection p <- normalize(max(p - q_c, 0)) and the
 *    next child is tested.  When every child is rejected the extra token is drawn from that
 *    residual p; at a node without children it is drawn from the node's target distribution.
 *    The paper takes the children in random order; for children drawn independently each
 *    stage's law needs only that the tested child is drawn from its own q, so any fixed order is
 *    exact and the caller's order is used;
 *  - Rule 1 (T = 0): the first child (ascending node order) whose token equals the target argmax at
 *    the current node (ties to the smallest id) is accepted; when none does, the extra token is that
 *    argmax;
 *  - uniforms: r_c is word 0 of the Philox block keyed (seed; counter (c, i, 0, 0)), the node's
 *    own index taking the place of the position; the extra token's u is word 1 of the block of the
 *    target row it is drawn from (0 at the root, n + 1 after node n).  On a chain both are the
 *    linear draft's;
 *  - a residual with S = 0 (impossible in exact arithmetic after a rejection) restarts from the
 *    current node's target distribution;
 *  - bad requests (accepted_len -1, every slot -1): a token outside [0, V), a parent outside
 *    [-1, n - 1], a draft row index outside [0, n_draft_rows), a temperature that describes no
 *    profile, and at T > 0 a node whose draft probability at its own token is zero.
 * Outputs: accepted_len[i] = a, the depth of the accepted path; out_tokens[cu[i] + i + d] for
 * d < a the path's tokens, then the extra token, then -1 up to slot N_i; accepted_nodes[cu[i] + d]
 * for d < a the path's node indices, then -1 up to N_i - 1.  diag: target_lse / draft_lse of
 * every row, ratio and accept_margin at the nodes tested (NaN elsewhere), cdf_margin, terminal_kind,
 * and resid_mass = the product of the stage masses S of the draw's residual (1 for a bonus).
 */
static void verify_tree_request(const void* target, const void* draft, int dtype, const int32_t* tokens,
                                const int32_t* parents, const int32_t* draft_row, int64_t n_draft_rows,
                                const int32_t* cu, int32_t i, int64_t n_nodes, int32_t V, double T, uint64_t seed,
                                int32_t* accepted_len, int32_t* out_tokens, int32_t* accepted_nodes, oracle_diag* dg,
                                double* p, double* q) {
  const int64_t lo = cu[i], hi = cu[i + 1];
  const int64_t N = hi - lo;
  if (dg && dg->cdf_margin) dg->cdf_margin[i] = NAN;
  if (dg && dg->resid_mass) dg->resid_mass[i] = NAN;
  if (lo < 0 || hi > n_nodes || N < 0 || N > ORACLE_MAX_DEPTH) { /* no slot can be named */
    accepted_len[i] = -1;
    if (dg && dg->terminal_kind) dg->terminal_kind[i] = ORACLE_TERM_BAD;
    return;
  }
  const int64_t trow0 = lo + i, drow0 = lo;
  int32_t* slots = out_tokens + trow0;
  int32_t* path = accepted_nodes + drow0; /* [N]: the accepted nodes, then -1 */
  for (int64_t d = 0; d < N; ++d) path[d] = -1;
  for (int64_t d = 0; d <= N; ++d) slots[d] = -1;
  if (dg) {
    for (int64_t n = 0; n < N; ++n) {
      set_nan(dg->ratio ? &dg->ratio[drow0 + n] : NULL);
      set_nan(dg->accept_margin ? &dg->accept_margin[drow0 + n] : NULL);
    }
  }

  int bad = !(T >= 0.0) || isinf(T);
  int64_t qrow[ORACLE_MAX_DEPTH]; /* the draft row of each node */
  for (int64_t n = 0; n < N && !bad; ++n) {
    const int32_t x = tokens[drow0 + n], par = parents[drow0 + n];
    qrow[n] = draft_row ? draft_row[drow0 + n] : drow0 + n;
    if (x < 0 || x >= V || par < -1 || par >= n || qrow[n] < 0 || qrow[n] >= n_draft_rows) bad = 1;
  }
  double lse_t[ORACLE_MAX_DEPTH + 1], lse_d[ORACLE_MAX_DEPTH];
  if (!bad && T > 0.0) {
    for (int64_t r = 0; r <= N; ++r) lse_t[r] = oracle_row_lse(target, dtype, trow0 + r, V, T);
    for (int64_t n = 0; n < N; ++n) {
      lse_d[n] = oracle_row_lse(draft, dtype, qrow[n], V, T);
      if (logit_at(draft, dtype, qrow[n], V, tokens[drow0 + n]) == -INFINITY) bad = 1; /* q_n(x_n) = 0 */
    }
  }
  if (bad) {
    accepted_len[i] = -1;
    if (dg && dg->terminal_kind) dg->terminal_kind[i] = ORACLE_TERM_BAD;
    return;
  }

  int64_t a = 0;
  int64_t u = -1; /* the current node; -1 is the root, whose target row is 0 */
  int32_t y;
  int kind;
  if (T == 0.0) { /* ---- Rule 1 */
    for (;;) {
      const int32_t g = oracle_row_argmax(target, dtype, trow0 + u + 1, V);
      if (dg && dg->target_argmax) dg->target_argmax[trow0 + u + 1] = g;
      int64_t next = -1;
      for (int64_t c = u + 1; c < N && next < 0; ++c) /* a child's index exceeds its parent's */
        if (parents[drow0 + c] == u && tokens[drow0 + c] == g) next = c;
      if (next < 0) {
        y = g;
        break;
      }
      path[a++] = (int32_t)next;
      u = next;
    }
    kind = ORACLE_TERM_GREEDY;
  } else { /* ---- Rule 2 */
    if (dg) {
      for (int64_t r = 0; r <= N; ++r)
        if (dg->target_lse) dg->target_lse[trow0 + r] = lse_t[r];
      for (int64_t n = 0; n < N; ++n)
        if (dg->draft_lse) dg->draft_lse[drow0 + n] = lse_d[n];
    }
    for (;;) {
      const int64_t row = u + 1; /* the current node's target row within the request */
      for (int32_t v = 0; v < V; ++v) p[v] = exp(logit_at(target, dtype, trow0 + row, V, v) / T - lse_t[row]);
      int rejected = 0, empty = 0;
      int pending = 0;   /* p holds the last residual unnormalized, its total S_last */
      double S_last = 1.0;
      double mass = 1.0; /* product of the earlier stages' masses */
      int64_t next = -1;
      for (int64_t c = u + 1; c < N && next < 0; ++c) {
        if (parents[drow0 + c] != u) continue;
        if (pending) { /* normalize(max(p - q, 0)) */
          for (int32_t v = 0; v < V; ++v) p[v] /= S_last;
          mass *= S_last;
          pending = 0;
        }
        const int32_t x = tokens[drow0 + c];
        for (int32_t v = 0; v < V; ++v) q[v] = exp(logit_at(draft, dtype, qrow[c], V, v) / T - lse_d[c]);
        /* the first child sees the node's own p: its ratio in the log form of the linear walk */
        const double ratio =
            rejected ? p[x] / q[x]
                     : exp((logit_at(target, dtype, trow0 + row, V, x) - logit_at(draft, dtype, qrow[c], V, x)) / T -
                           (lse_t[row] - lse_d[c]));
        uint32_t blk[4];
        oracle_philox_block(seed, (uint32_t)i, (uint32_t)c, blk);
        const double r = accept_uniform(blk);
        if (dg && dg->ratio) dg->ratio[drow0 + c] = ratio;
        if (dg && dg->accept_margin) dg->accept_margin[drow0 + c] = fabs(r - ratio);
        if (r <= ratio) {
          next = c;
          break;
        }
        double S = 0.0;
        for (int32_t v = 0; v < V; ++v) {
          p[v] = p[v] > q[v] ? p[v] - q[v] : 0.0;
          S += p[v];
        }
        rejected = 1;
        if (S > 0.0) {
          pending = 1;
          S_last = S;
          empty = 0;
        } else { /* restart from the node's target distribution */
          for (int32_t v = 0; v < V; ++v) p[v] = exp(logit_at(target, dtype, trow0 + row, V, v) / T - lse_t[row]);
          pending = 0;
          mass = 1.0;
          empty = 1;
        }
      }
      if (next >= 0) {
        path[a++] = (int32_t)next;
        u = next;
        continue;
      }
      uint32_t blk[4];
      oracle_philox_block(seed, (uint32_t)i, (uint32_t)row, blk);
      double S, margin;
      y = inverse_cdf(p, V, draw_uniform(blk), &S, &margin); /* normalizes a pending residual itself */
      kind = !rejected ? ORACLE_TERM_BONUS : (empty ? ORACLE_TERM_RESIDUAL_EMPTY : ORACLE_TERM_RESIDUAL);
      if (dg && dg->cdf_margin) dg->cdf_margin[i] = margin;
      if (dg && dg->resid_mass) dg->resid_mass[i] = mass * S;
      break;
    }
  }
  for (int64_t d = 0; d < a; ++d) slots[d] = tokens[drow0 + path[d]];
  slots[a] = y;
  accepted_len[i] = (int32_t)a;
  if (dg && dg->terminal_kind) dg->terminal_kind[i] = kind;
}

/*
 * Token-tree batches (see above).  target [n_nodes + B][V], draft [n_draft_rows][V] (may be NULL
 * when T == 0), draft_tokens and parents [n_nodes], draft_row [n_nodes] each node's draft row (NULL:
 * node cu[i] + n takes row cu[i] + n, and n_draft_rows must be n_nodes), cu [B + 1] node offsets,
 * accepted_len [B], out_tokens [n_nodes + B], accepted_nodes [n_nodes].  Returns 0, or -1 for
 * arguments that describe no batch.
 */
int oracle_verify_tree(const void* target, const void* draft, int dtype, const int32_t* draft_tokens,
                       const int32_t* parents, const int32_t* draft_row, int64_t n_draft_rows, const int32_t* cu,
                       int32_t B, int64_t n_nodes, int32_t V, double T, uint64_t seed, int32_t* accepted_len,
                       int32_t* out_tokens, int32_t* accepted_nodes, oracle_diag* diag) {
  if (!target || !draft_tokens || !parents || !cu || !accepted_len || !out_tokens || !accepted_nodes) return -1;
  if (B <= 0 || V <= 0 || n_nodes < 0 || !(T >= 0.0) || isinf(T) || (T > 0.0 && !draft && n_nodes > 0)) return -1;
  if (n_draft_rows < 0 || (!draft_row && n_draft_rows != n_nodes)) return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP32) return -1;
  int failed = 0;
#pragma omp parallel reduction(| : failed)
  {
    double* p = (double*)malloc(sizeof(double) * 2 * (size_t)V);
    if (!p) failed = 1;
#pragma omp for schedule(dynamic, 1)
    for (int32_t i = 0; i < B; ++i)
      if (p)
        verify_tree_request(target, draft, dtype, draft_tokens, parents, draft_row, n_draft_rows, cu, i, n_nodes, V,
                            T, seed, accepted_len, out_tokens, accepted_nodes, diag, p, p + V);
    free(p);
  }
  return failed ? -2 : 0;
}

/* Number of OpenMP threads the oracle runs on (for reporting), and a way to change it (timing). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif
