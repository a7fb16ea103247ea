/*
 * sdv.h -- C ABI of the MI355X (gfx950) speculative-decoding verification library (libsdv.so).
 *
 * The library verifies a batch of draft proposals against target logits in one call, on one GPU,
 * with hand-written HIP kernels.  Every pointer argument of sdv_verify / sdv_verify_ex /
 * sdv_philox4x32_10 is a DEVICE pointer owned by the caller; the library never allocates, frees,
 * copies to the host or synchronizes.  All work is enqueued on the caller's HIP stream and the call
 * returns as soon as it is enqueued.  Calls are stateless and may run concurrently on different
 * streams as long as they use different workspaces and outputs.
 *
 * Definitions the entry points follow:
 *  - Rule 1 (temperature 0) and Rule 2 (temperature > 0) of "Speculative Decoding Coordination
 *    Protocol (SDCP)", section "Acceptance Rules"; the accept test r <= p(x)/q(x) of "SOTA-227:
 *    Decode with a draft model and an accept-reject rule, which is exactly lossless", section
 *    "What to do".  p and q are softmax(z/T) of the target and draft logit rows, truncated by
 *    top-k and top-p when sdv_options carries them (SDCP section "Session Contract": the sampling
 *    profile applies temperature, then top-k, then top-p).
 *  - Ragged batches ("M7.8 - Speculative Serving", section 0x00, background on the serving unit,
 *    N_query = sum_i (K_i + 1)):
 *    request i has K_i = cu[i+1] - cu[i] draft tokens, 0 <= K_i <= 64 (SDCP m_max <= 64).
 *    Draft row of (i, j), j < K_i:  row cu[i] + j        of draft_logits / draft_tokens.
 *    Target row of (i, j), j <= K_i: row cu[i] + i + j   of target_logits.
 *  - Uniforms: Philox4x32-10 (Salmon et al., SC'11), key = (seed low 32 bits, seed high 32 bits),
 *    counter = (position j, request i, 0, 0).  Accept test r = ((w0 >> 8) + 1) * 2^-24 in (0, 1];
 *    correction / bonus draw u = (w1 >> 8) * 2^-24 in [0, 1), from the block of the drawn position.
 *  - The correction (first rejected position t) is drawn from normalize(max(p_t - q_t, 0)); if no
 *    position is rejected the bonus is drawn from p at position K_i.  The draw is the inverse CDF
 *    in ascending token id: y = min{v : C(v) > u * S}, S the total weight.
 */
#ifndef SDV_H
#define SDV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDV_ABI_VERSION 5
#define SDV_MAX_DEPTH 64 /* largest K_i a request may carry */
#define SDV_MAX_EVENTS 4 /* timing hooks in sdv_diag */

typedef enum { SDV_BF16 = 0, SDV_FP32 = 1 } sdv_dtype;

typedef enum {
  SDV_OK = 0,
  SDV_ERR_INVALID_ARG = -1, /* a required pointer is NULL, or a size / temperature is out of range */
  SDV_ERR_UNSUPPORTED = -2, /* dtype not one of sdv_dtype */
  SDV_ERR_LIMIT = -3,       /* the batch exceeds an index or launch-size limit of the library */
  SDV_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than sdv_workspace_bytes() */
  SDV_ERR_HIP = -5          /* a kernel launch failed; the stream state is as HIP reports it */
} sdv_status;

/* Terminal kinds reported through sdv_diag.terminal_kind. */
typedef enum {
  SDV_TERM_GREEDY = 0,         /* temperature 0: the extra token is the target argmax */
  SDV_TERM_BONUS = 1,          /* every draft accepted (or K_i = 0): drawn from p at position K_i */
  SDV_TERM_RESIDUAL = 2,       /* first rejection at t < K_i: drawn from max(p_t - q_t, 0) */
  SDV_TERM_RESIDUAL_EMPTY = 3, /* the residual had no positive weight in floating point: drawn from p_t */
  SDV_TERM_NONE = 4,           /* a stop token or the budget ended emission inside the accepted drafts:
                                  no extra token is emitted or drawn (sdv_verify_opts) */
  SDV_TERM_BAD = -1            /* the request was rejected (see sdv_verify) */
} sdv_terminal_kind;

/*
 * Optional diagnostics for sdv_verify_ex.  Every member may be NULL; non-NULL arrays are device
 * pointers the library writes for valid requests only (other entries are left untouched).
 *   target_lse     [n_draft_rows + B]  ln sum_v exp(z_v / T) of each target row      (T > 0)
 *   draft_lse      [n_draft_rows]      ln sum_v exp(z_v / T) of each draft row       (T > 0)
 *   target_argmax  [n_draft_rows + B]  argmax of each target row, smallest id on ties (T == 0)
 *   ratio          [n_draft_rows]      p_j(x_j) / q_j(x_j) at every draft position   (T > 0)
 *   accept_uniform [n_draft_rows]      r_j at every draft position                   (T > 0)
 *   draw_uniform   [B]                 u of the drawn position                        (T > 0)
 *   terminal_kind  [B]                 one of sdv_terminal_kind
 *   events         hipEvent_t handles (cast to void*) recorded on the stream: events[0] before the
 *                  first kernel, events[1] after the row pass (one record per 16 KiB chunk of
 *                  every row read), events[3] after the truncation kernel (top-k / top-p through
 *                  sdv_verify_opts; not recorded when it does not run), events[2] after the verdict
 *                  kernel (per request: fold, accept scan, terminal draw).  A batch of one request
 *                  with 16-byte aligned rows of at most 15 chunks in all, one profile and no
 *                  truncation or probability rows, runs both passes in one launch: events[1] and
 *                  events[2] are then both recorded after it.
 *   target_logit   [n_draft_rows]      z_target[x_j], the stored target logit at each draft token,
 *                                      widened to binary32 (T > 0)
 *   draft_logit    [n_draft_rows]      z_draft[x_j], the same on the draft row (T > 0, draft logits;
 *                                      with sdv_options.draft_probs it holds q_j(x_j) as given)
 *   terminal_mass  [B]                 S, the total weight of the extra-token draw in probability
 *                                      units: sum_v max(p_t(v) - q_t(v), 0) for a correction, the
 *                                      mass of p_K (1 up to rounding) for a bonus or for a draw from
 *                                      p_t after an empty residual (T > 0, requests that draw)
 * The gathers and S are the quantities the accept test and the inverse CDF are built from (SDCP
 * "Acceptance Rules", Rule 2: p_i(x_i)/q_i(x_i) and normalize(max(p - q, 0))).
 */
typedef struct sdv_diag {
  double* target_lse;
  double* draft_lse;
  int32_t* target_argmax;
  double* ratio;
  float* accept_uniform;
  float* draw_uniform;
  int32_t* terminal_kind;
  void* events[SDV_MAX_EVENTS];
  float* target_logit;
  float* draft_logit;
  double* terminal_mass;
} sdv_diag;

/*
 * Bytes of device workspace sdv_verify needs for a batch of this shape (0 on invalid shapes).
 * The workspace needs no initialisation and holds nothing between calls.  It holds 8 bytes per
 * chunk of every logit row (16 KiB of logits) and 8 bytes per row; bf16 batches add 260 bytes per
 * chunk, where the row pass of a top-k / top-p call counts the logits just below each chunk's
 * maximum, and 4 bytes per row.  Each request adds 8 bytes per chunk of a row and 4 bytes, where
 * the verdict workgroups that share a correction publish its residual masses.
 */
size_t sdv_workspace_bytes(int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype);

/*
 * Verify one ragged batch (SDCP "Verification and Commit", steps 5 to 7, for every request).
 *
 *   target_logits  [n_draft_rows + B][V] row-major, dtype elements (bf16 as raw 16-bit words),
 *                                        the base aligned to the element size (2 or 4 bytes); rows
 *                                        that are 16-byte aligned (base and V * size) take the
 *                                        fastest loads, any other V costs a few element loads a chunk
 *   draft_logits   [n_draft_rows][V]     same dtype and alignment; may be NULL when temperature == 0
 *                                        (it is not read then) or when n_draft_rows == 0
 *   draft_tokens   [n_draft_rows] int32  the proposed token of each draft position
 *   ragged_offsets [B + 1] int32         cu[0] = 0, non-decreasing, cu[B] = n_draft_rows
 *   B, n_draft_rows, V                   host values: B >= 1, n_draft_rows >= 0, V >= 1
 *   dtype                                SDV_BF16 or SDV_FP32
 *   temperature                          0 selects Rule 1 (greedy); > 0 selects Rule 2 with
 *                                        p = softmax(z_target / T), q = softmax(z_draft / T)
 *   seed                                 key of the verifier's Philox stream (vary it per round)
 *   accepted_len   [B] int32 out         a_i in [0, K_i] accepted drafts, or -1 for a rejected request
 *   out_tokens     [n_draft_rows + B] int32 out: request i writes slots cu[i]+i .. cu[i]+i+K_i:
 *                                        its a_i accepted drafts, then the correction / bonus
 *                                        token, then -1 in the remaining K_i - a_i slots
 *   workspace      device scratch of at least sdv_workspace_bytes(...) bytes, 256-byte aligned
 *   stream         hipStream_t (as void*), NULL for the null stream
 *
 * Errors.  Argument errors are detected on the host and returned synchronously; nothing is
 * launched then: NULL required pointers, logits not aligned to their element size, B < 1,
 * n_draft_rows < 0, V < 1, temperature negative, NaN or infinite (or so small that log2(e)/T
 * overflows), T > 0 with NULL draft_logits while n_draft_rows > 0 -> SDV_ERR_INVALID_ARG; unknown dtype -> SDV_ERR_UNSUPPORTED; sizes beyond the
 * 32-bit row / launch limits -> SDV_ERR_LIMIT; small workspace -> SDV_ERR_WORKSPACE.
 * Per-request errors are decided on the device before any uniform is used (SDCP step 5 and
 * problem types "sdcp-bad-proposal" / "sdcp-limit"): a request whose depth is outside [0, 64] or
 * whose offsets fall outside [0, n_draft_rows] gets accepted_len = -1 and none of its slots are
 * written; a request with a draft token outside [0, V), or (T > 0) with a draft logit of -inf at
 * its token (q = 0), gets accepted_len = -1 and all of its K_i + 1 slots set to -1.  Other requests
 * are unaffected.  Launch failures -> SDV_ERR_HIP.
 */
int sdv_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
               const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
               double temperature, uint64_t seed, int32_t* accepted_len, int32_t* out_tokens,
               void* workspace, size_t workspace_bytes, void* stream);

/* sdv_verify plus optional diagnostics and timing events (diag may be NULL). */
int sdv_verify_ex(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                  const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                  double temperature, uint64_t seed, int32_t* accepted_len, int32_t* out_tokens,
                  void* workspace, size_t workspace_bytes, void* stream, const sdv_diag* diag);

/*
 * sdv_verify_ex with a sampling profile per request.  SDCP ("Speculative Decoding Coordination
 * Protocol (SDCP)") fixes a sampling profile per session (section "Session Contract"; section
 * "Sampling Policy Updates" lets it change between rounds), and one verification batch gathers
 * requests of many sessions, so temperature and seed come per request:
 *
 *   temperature  [B] float device array: T_i = 0 selects Rule 1 for request i, T_i > 0 Rule 2 with
 *                p = softmax(z_target / T_i), q = softmax(z_draft / T_i)
 *   seed         [B] uint64 device array: the Philox key of request i (counter as in sdv_verify)
 *
 * Everything else is as in sdv_verify_ex.  draft_logits must be non-NULL whenever
 * n_draft_rows > 0 (draft rows of greedy requests are not read).  A temperature that is negative,
 * NaN, infinite, or so small that log2(e)/T_i overflows binary32 describes no profile: that request
 * gets accepted_len = -1 and all of its K_i + 1 slots set to -1, and the other requests are
 * unaffected.  NULL temperature or seed -> SDV_ERR_INVALID_ARG.
 */
int sdv_verify_profiled(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                        const float* temperature, const uint64_t* seed, int32_t* accepted_len, int32_t* out_tokens,
                        void* workspace, size_t workspace_bytes, void* stream, const sdv_diag* diag);

/*
 * Per-request options of sdv_verify_opts.  Every member may be NULL (n_stop_tokens 0), which keeps
 * the behaviour of sdv_verify_ex; all arrays are DEVICE arrays owned by the caller.
 *
 *  temperature, seed  [B] float / uint64: one sampling profile per request, as in
 *                     sdv_verify_profiled (both or neither; they replace the scalar T and seed).
 *  accept_uniform     [n_draft_rows] double: the caller's r in [0, 1) for each draft position.
 *  draw_uniform       [n_draft_rows + B] double: the caller's u in [0, 1) for each position, in the
 *                     target-row layout (position j of request i at cu[i] + i + j).
 *                     Both or neither.  With them the uniforms come from the caller instead of
 *                     Philox (for instance SDCP's HMAC-SHA-256 values, sdv_sdcp_uniforms), and the
 *                     accept test is SDCP Rule 2's strict one, r < p/q ("Speculative Decoding
 *                     Coordination Protocol (SDCP)", section "Acceptance Rules").  Values outside
 *                     [0, 1) give unspecified (memory-safe) verdicts.
 *  stop_offsets       [B + 1] int32, stop_tokens [n_stop_tokens] int32: request i stops at any token
 *                     of stop_tokens[stop_offsets[i] .. stop_offsets[i + 1]).  A list outside
 *                     [0, n_stop_tokens] rejects that request (accepted_len -1, every slot -1).
 *  budget             [B] int32: the remaining output budget of each request (<= 0 emits nothing).
 *  emitted_len        [B] int32 out: the number of tokens request i emits.
 *  top_k, top_p_milli [B] int32: the rest of each request's sampling profile (SDCP section
 *                     "Session Contract": top_k a count, top_p_milli the nucleus mass in thousandths).
 *                     At T > 0, p and (from draft logits) q are truncated after the temperature:
 *                     tokens rank by probability, equal probabilities going to the smaller token
 *                     id; top-k keeps the first top_k ranks; top-p then keeps the shortest run of
 *                     leading ranks whose mass, renormalised over the top-k set, reaches
 *                     top_p_milli / 1000, and never fewer than one token; the kept tokens are
 *                     renormalised.  top_k 0 (or >= V) and top_p_milli 1000 truncate nothing; a
 *                     negative value or top_p_milli > 1000 describes no profile and rejects the
 *                     request (accepted_len -1, every slot -1).  A draft token outside the kept
 *                     set of its draft row has q = 0 and rejects the request before any uniform
 *                     is used.  Given q rows (draft_probs) are not truncated.  Rule 1 (T = 0) keeps
 *                     its argmax under any truncation and ignores both.  Either may be NULL.
 *  kept_tokens        [n_draft_rows + B + n_draft_rows] int32 out (with top_k or top_p_milli): the
 *                     number of tokens each row keeps, target rows first, then draft rows (V for a
 *                     row that is not truncated); written for the rows of requests at T > 0 (draft
 *                     rows only when draft logits are used).
 *  draft_probs        [n_draft_rows][V] float (binary32, 4-byte aligned): the draft distributions, SDCP's
 *                     "q_rows" (section "Message Definitions"; Rule 2 takes q[i] from them), used as
 *                     given in place of softmax(draft_logits / T); draft_logits is then not read and
 *                     may be NULL.  Each row must be the distribution the token was drawn from (sums
 *                     to 1 up to rounding).  A q that is not positive at the proposed token rejects
 *                     the request before any uniform is used (SDCP "Verification and Commit", step
 *                     5).  The row pass then streams target rows only; q is read at the proposed
 *                     tokens and, for a correction, over the rejected position's row.
 *  verdict_split      workgroups per request in the verdict pass (0: chosen from B and V; values
 *                     above the number of 16 KiB chunks per row count as that number; negative ->
 *                     SDV_ERR_INVALID_ARG).  The workgroups of a request share a correction's pass
 *                     over the rejected position's rows; every chunk's residual mass is computed
 *                     the same way whichever workgroup computes it, so no output depends on the
 *                     value.  A performance setting, not part of the method.
 *
 * Emission (SDCP section "Verification and Commit", step 7; "M7.8 - Speculative Serving", section
 * 0x09, "EOS and length-limit stopping"): of the a_i + 1 candidate tokens (the accepted drafts,
 * then the extra token), no token after the first stop token and no more than budget[i] are
 * emitted; out_tokens holds the emitted tokens first and -1 in every other slot of the request.
 * accepted_len still reports a_i.  When emission ends inside the accepted drafts the extra token is
 * neither emitted nor drawn (terminal kind SDV_TERM_NONE).  A rejected request emits 0 tokens.
 */
typedef struct sdv_options {
  const float* temperature;
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
  int32_t verdict_split;
} sdv_options;

/*
 * sdv_verify_ex refined by per-request options (options may be NULL).  With options->temperature
 * the scalar temperature and seed are ignored and draft_logits must be non-NULL when
 * n_draft_rows > 0.  Errors as in sdv_verify_ex, plus SDV_ERR_INVALID_ARG for a uniform array
 * without its partner, a temperature array without seeds (or the reverse), or stop_offsets with
 * n_stop_tokens < 0 or (n_stop_tokens > 0 and stop_tokens NULL).
 */
int sdv_verify_opts(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                    const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                    double temperature, uint64_t seed, const sdv_options* options, int32_t* accepted_len,
                    int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream,
                    const sdv_diag* diag);

/*
 * Verification of token trees: multi-step speculative sampling over a tree of drafts (Miao et al.,
 * "SpecInfer: Accelerating Large Language Model Serving with Tree-based Speculative Inference and
 * Verification", ASPLOS 2024, section 4, the token tree verifier).  The pages define no tree rule
 * (SDCP section "Scope" leaves tree-structured speculation out of its first version); Rules 1 and 2
 * of SDCP "Acceptance Rules" are applied node by node as follows.
 *
 * Request i holds N_i = cu[i + 1] - cu[i] <= 64 nodes n = 0 .. N_i - 1 (ragged_offsets as for
 * linear drafts).  All arrays are DEVICE arrays:
 *   parents       [n_nodes] int32   node n's parent within its request, in [-1, n - 1] (-1: the
 *                                   root, the last committed token); nodes come in an order where
 *                                   every parent precedes its children
 *   draft_tokens  [n_nodes] int32   node n's token
 *   target_logits [n_nodes + B][V]  row cu[i] + i at the root, cu[i] + i + n + 1 after node n
 *   draft_row     [n_nodes] int32   node n's draft row, in [0, n_draft_rows) (siblings from one
 *                                   drafter share their parent context's row); NULL: node cu[i] + n
 *                                   takes row cu[i] + n, and n_draft_rows must equal n_nodes
 *   draft_logits  [n_draft_rows][V] the logits the nodes' tokens were drawn from (at each node's
 *                                   parent's context), n_draft_rows <= n_nodes; may be NULL when
 *                                   temperature == 0
 * A chain (every node the parent of the next) is exactly a linear draft of sdv_verify, with the
 * same uniforms and results.
 *   T > 0: at the current node (the root first), with p its target distribution softmax(z / T),
 *          the children are tested in node order: child c is accepted iff r_c <= p(x_c) / q_c(x_c)
 *          with q_c = softmax(draft row of c / T), and the walk moves to c; a rejection replaces p
 *          by normalize(max(p - q_c, 0)) and the next child is tested.  When every child is
 *          rejected the extra token is drawn from that p; at a node without children it is drawn
 *          from the node's own target distribution.  r_c: word 0 of the Philox block keyed (seed;
 *          counter (c, i, 0, 0)); the draw: word 1 of the block of the target row it is drawn from
 *          (0 at the root, n + 1 after node n), by the inverse CDF in ascending token id.
 *   T = 0: the first child (node order) whose token equals the target argmax of the current node
 *          (ties to the smallest id) is accepted; when none does, that argmax is the extra token.
 * Outputs: accepted_len [B] the depth a of the accepted path; out_tokens [n_nodes + B] the path's
 * tokens at cu[i] + i .. cu[i] + i + a - 1, the extra token at cu[i] + i + a, -1 up to
 * cu[i] + i + N_i; accepted_nodes [n_nodes] the path's node indices (within the request) at
 * cu[i] .. cu[i] + a - 1, -1 up to cu[i] + N_i - 1.
 * Bad requests (accepted_len -1, every slot -1): a token outside [0, V), a parent outside
 * [-1, n - 1], at T > 0 a draft row index outside [0, n_draft_rows) or a node whose draft logit at
 * its own token is -inf (q = 0).  Offsets that
 * are not valid, or a request of more than 64 nodes, reject without writing slots, as sdv_verify.
 * workspace: sdv_workspace_bytes(B, n_nodes, V, dtype).  diag (may be NULL): target_lse,
 * draft_lse, target_logit / draft_logit (z_t at the parent's row and z_d at each node's token),
 * ratio and accept_uniform at the nodes tested (others untouched), target_argmax of the rows
 * visited (T = 0), draw_uniform, terminal_kind, terminal_mass (the residual's mass in probability
 * units, M = product of the stage masses; about 1 for a bonus) and the events (row pass, verdicts).
 * Per-request profiles, truncation, stop lists and caller uniforms are not taken on this path.
 * Errors as sdv_verify; NULL parents, draft_tokens or accepted_nodes with n_nodes > 0, n_draft_rows
 * outside [0, n_nodes] (or other than n_nodes without draft_row), or T > 0 with n_draft_rows > 0 and
 * NULL draft_logits -> SDV_ERR_INVALID_ARG.  A rejected sibling that shares the previous rejected
 * sibling's draft row costs its residual pass no extra row: consecutive rejections on one row are
 * applied to one load of it.
 */
int sdv_verify_tree(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                    const int32_t* parents, const int32_t* draft_row, const int32_t* ragged_offsets, int32_t B,
                    int64_t n_nodes, int64_t n_draft_rows, int32_t V, int32_t dtype, double temperature,
                    uint64_t seed, int32_t* accepted_len, int32_t* accepted_nodes, int32_t* out_tokens,
                    void* workspace, size_t workspace_bytes, void* stream, const sdv_diag* diag);

/*
 * SDCP's verifier uniforms, computed on the HOST for sdv_options ("Speculative Decoding
 * Coordination Protocol (SDCP)", section "Acceptance Rules", Rule 2).  For request i, with profile
 * seed seeds[i], session id sessions[16 i .. 16 i + 15] and round rounds[i], each value is the first
 * 53 bits of HMAC-SHA-256 keyed with the seed as eight octets in network byte order over
 *   "SDCP-VERIFY-1" || 0x00 || session || uint32(round) || uint32(position) || uint8(purpose)
 * (integers in network byte order; positions counted from 1 as SDCP numbers p[1..M+1]), divided by
 * 2^53.  Purpose 0 feeds the acceptance test, purpose 1 the draw of the extra token.  Writes
 *   accept_uniform[cu[i] + j]      purpose 0 at position j + 1, j < K_i   (HOST, cu[B] doubles)
 *   draw_uniform[cu[i] + i + t]    purpose 1 at position t + 1, t <= K_i  (HOST, cu[B] + B doubles)
 * cu is a HOST copy of the ragged offsets.  Invalid offsets (cu[0] != 0, decreasing, a depth above
 * 64) or NULL pointers -> SDV_ERR_INVALID_ARG and nothing written.
 */
int sdv_sdcp_uniforms(int32_t B, const int32_t* cu, const uint64_t* seeds, const uint8_t* sessions,
                      const uint32_t* rounds, double* accept_uniform, double* draw_uniform);

/*
 * Post-verification commit of a batch ("M7.8 - Speculative Serving", sections 0x03C and 0x03D:
 * the ragged results are unpadded and each request's emitted tokens appended to its logical
 * sequence at contiguous positions; section 0x09 for the lengths after a round).  All arrays are
 * DEVICE arrays; ragged_offsets, accepted_len and out_tokens are those of the verification call,
 * emitted_len its sdv_options.emitted_len (NULL: every valid request emitted a_i + 1 tokens), and
 * prefix_len [B] int32 each request's logical length P_i before the round.  Writes:
 *   new_offsets   [B + 1]            exclusive prefix sums of the emitted counts n_i
 *   new_tokens    [n_draft_rows + B] request i's emitted tokens at new_offsets[i] ..
 *   new_positions [n_draft_rows + B] their logical positions P_i, P_i + 1, ...
 *   lengths       [B][3]             (L_out, L_target, L_draft) = (P + E + F, P + E,
 *                                    P + min(E, max(K - 1, 0))), E the accepted drafts emitted and
 *                                    F = 1 when the extra token was emitted
 *   next_token, next_position [B]    the last emitted token and its position, or -1 when none
 * A rejected request (accepted_len -1) or one whose offsets fall outside [0, n_draft_rows] emits
 * nothing.  With offsets that are not non-decreasing the counts can sum past n_draft_rows + B:
 * new_offsets reports them as they are, and no token is written beyond the arrays.  Errors: B < 1,
 * n_draft_rows < 0 or a NULL required pointer -> SDV_ERR_INVALID_ARG; n_draft_rows + B above
 * INT32_MAX -> SDV_ERR_LIMIT.
 */
int sdv_commit(int32_t B, int64_t n_draft_rows, const int32_t* ragged_offsets, const int32_t* accepted_len,
               const int32_t* emitted_len, const int32_t* out_tokens, const int32_t* prefix_len, int32_t* new_offsets,
               int32_t* new_tokens, int32_t* new_positions, int32_t* lengths, int32_t* next_token,
               int32_t* next_position, void* stream);

/*
 * The repadded form of a verified batch ("M7.8 - Speculative Serving", section 0x03D: the unpadded
 * results are appended to each request's logical sequence and the batch is padded again to a
 * rectangle; section 0x03C's position invariant: the non-padding tokens of a row sit at logical
 * positions 0 .. L - 1 and padding takes no position).  All arrays are DEVICE arrays.
 * ragged_offsets, accepted_len, out_tokens and emitted_len are as for sdv_commit; prefix_offsets
 * [B + 1] and prefix_tokens [n_prefix_tokens] hold each request's logical sequence before the round
 * in CSR form (request i: prefix_tokens[prefix_offsets[i] .. prefix_offsets[i + 1] - 1]).  Row i of
 * the [B][width] outputs holds that prefix followed by the request's emitted tokens, L_i tokens in
 * all, at positions 0 .. L_i - 1:
 *   token_ids    [B][width] int32   the tokens, pad_id in padding cells
 *   position_ids [B][width] int32   logical positions, -1 in padding cells
 *   mask         [B][width] uint8   1 for a token, 0 for padding
 *   row_len      [B]        int32   L_i
 * left_pad != 0 puts the padding before the tokens (every row ends in the last column), 0 after.
 * The section's width is the longest L_i (lengths[3 i] of sdv_commit); a row with L_i > width is
 * written as padding only and reports L_i, so the caller can see it did not fit.  A row whose
 * prefix offsets decrease or fall outside [0, n_prefix_tokens] is padding only and reports -1; a
 * rejected request (accepted_len -1) keeps its prefix unchanged.  No KV block table is produced.
 * Errors: B < 1, n_draft_rows < 0, n_prefix_tokens < 0, width < 1, or a NULL required pointer
 * (prefix_tokens may be NULL when n_prefix_tokens is 0) -> SDV_ERR_INVALID_ARG; n_draft_rows + B
 * above INT32_MAX, n_prefix_tokens above INT32_MAX - 128 or B * width above 2^40 -> SDV_ERR_LIMIT.
 */
int sdv_repad(int32_t B, int64_t n_draft_rows, const int32_t* ragged_offsets, const int32_t* accepted_len,
              const int32_t* emitted_len, const int32_t* out_tokens, const int32_t* prefix_offsets,
              const int32_t* prefix_tokens, int64_t n_prefix_tokens, int32_t width, int32_t pad_id, int32_t left_pad,
              int32_t* token_ids, int32_t* position_ids, uint8_t* mask, int32_t* row_len, void* stream);

/*
 * Raw Philox4x32-10 blocks on the device, for testing the verifier's uniforms: out[b] =
 * Philox4x32-10(counter = counters[b][0..3], key = keys[b][0..1]) for b < n.  counters [n][4],
 * keys [n][2], out [n][4] are uint32 device arrays.  n < 1 or NULL pointers -> SDV_ERR_INVALID_ARG.
 */
int sdv_philox4x32_10(const uint32_t* counters, const uint32_t* keys, int64_t n, uint32_t* out, void* stream);

/*
 * The verifier's own Philox blocks on the device, for testing its uniforms (the keying of sdv_verify:
 * key = (seed low 32 bits, seed high 32 bits), counter = (position j, request i, 0, 0); SDCP
 * "Acceptance Rules", Rule 2, one uniform per position and purpose: word 0 feeds the accept test,
 * word 1 the draw of the extra token).  Writes words[(i * P + j) * 4 + w] = word w of the block of
 * (request i, position j) for i < B, j < P: a uint32 device array of B * P * 4 words owned by the
 * caller.  B < 1, P < 1, NULL words -> SDV_ERR_INVALID_ARG; B * P above 2^31 - 1 -> SDV_ERR_LIMIT.
 */
int sdv_philox_uniforms(uint64_t seed, int32_t B, int32_t P, uint32_t* words, void* stream);

/*
 * Measurement hooks: the bandwidth yardsticks of the row pass.  Decoding is limited by memory
 * bandwidth, not arithmetic (SDCP, section "Introduction", its background paragraph; "SOTA-227",
 * section "Why it is free rather than a trade"); these kernels read n_chunks consecutive 16 KiB
 * chunks of src (device, 16-byte aligned, n_chunks * 16384 bytes) with no arithmetic, and write
 * out[c] (device uint32 [n_chunks]) = the xor of the 4096 words of chunk c.
 *   shape 0  the row pass's loads: 16-byte non-temporal register loads, one chunk per wave, four
 *            waves per workgroup (its rate is the best a read-once stream of the row pass's shape
 *            reaches)
 *   shape 1  direct-to-LDS loads, one chunk per wave, two waves per workgroup
 *   shape 2  register loads from a persistent grid (eight 256-thread workgroups per compute unit)
 *            whose waves stride over the chunks with two chunks in flight
 * sdv_read_ceiling is shape 0.  n_chunks < 1, a shape outside [0, 2], NULL or misaligned pointers ->
 * SDV_ERR_INVALID_ARG.
 */
int sdv_read_yardstick(const void* src, int64_t n_chunks, int32_t shape, uint32_t* out, void* stream);
int sdv_read_ceiling(const void* src, int64_t n_chunks, uint32_t* out, void* stream);

/*
 * sdv_verify for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The same verification as sdv_verify (same kernels,
 * same outputs) with no workspace argument: the library's scratch is a static device array of
 * SDV_NOALLOC_SCRATCH_BYTES bytes that each GPU the library runs on holds until the process ends (its
 * address is looked up once per device, on the first call with that device current).  The call
 * allocates and frees nothing.
 *   sdv_noalloc_bytes   the scratch a batch of this shape needs (0 on invalid shapes): 8 bytes per
 *                       16 KiB chunk of every row, 8 bytes per row, 8 bytes per chunk of a row and
 *                       4 bytes per request (no room for top-k / top-p counts: sdv_verify never
 *                       truncates), each array rounded up to 256 bytes.
 * Every call on one GPU shares that GPU's array and leaves its contents behind; each call clears
 * what it needs zeroed itself.  Calls that overlap in time on one GPU (on different streams) race on
 * the array: serialize them, for instance on one stream.  Errors as in sdv_verify, plus
 * SDV_ERR_LIMIT when sdv_noalloc_bytes(...) exceeds SDV_NOALLOC_SCRATCH_BYTES (nothing is launched)
 * and SDV_ERR_HIP when the current device cannot be queried or the array's address cannot be found.
 */
#define SDV_NOALLOC_SCRATCH_BYTES (8u << 20) /* 8 MiB per GPU */
size_t sdv_noalloc_bytes(int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype);
int sdv_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                       const int32_t* ragged_offsets, int32_t B, int64_t n_draft_rows, int32_t V, int32_t dtype,
                       double temperature, uint64_t seed, int32_t* accepted_len, int32_t* out_tokens, void* stream);

/* Human-readable name of a status code (static storage). */
const char* sdv_status_string(int status);

/* SDV_ABI_VERSION of the loaded library. */
int sdv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDV_H */
