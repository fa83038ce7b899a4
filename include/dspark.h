/*
 * dspark.h -- C ABI of the MI355X (gfx950) DSpark vocabulary-wide
 * propose / dyadic24 / verify library (libdspark.so).
 *
 * Definitions come from three public pages, cited by title and section:
 *   [Q]  "PP1 q transport and scheduling design", section "Distribution
 *        contract and precision" (the dyadic24 categorical q, its rejections,
 *        sparse top-k support, integer sampling) and section "Size and
 *        critical path" (dense / sparse q layouts and sizes).
 *   [C]  "Remote DSpark drafter -- wire and state contract (DSV41-OFFLOAD)",
 *        section 2 (greedy argmax with lowest-index ties; N = 5 block
 *        positions, anchor-as-first) and section 6.3 (draft_ids int32 and
 *        confidence float32 per request and position; failed entries carry
 *        id 0 and confidence 0.0; confidence must be finite in [0, 1]).
 *   [A]  "DeepSeek-V4.1 DSpark" (ROCm ATOM docs), section "State and
 *        sampling contracts" (greedy verification matches the target argmax
 *        over the anchor plus up to five proposals; the accepted prefix is
 *        committed).
 *
 * Conventions shared by every entry point
 *   Memory.   Every array argument is a DEVICE pointer owned by the caller
 *             (e.g. a torch tensor); struct arguments themselves are host
 *             memory.  The library never allocates or frees device memory.
 *             Logit rows are row-major, `row_stride` elements apart, and the
 *             first row and the row stride in bytes must be 16-byte aligned.
 *   Streams.  `stream` is a hipStream_t (NULL = the null stream).  Work is
 *             enqueued on it and the call returns without synchronising.
 *   Errors.   The host return value is DSPARK_SUCCESS (0) once the work is
 *             enqueued, or a negative DSPARK_E* code for a bad argument or a
 *             failed launch; on an argument error nothing is enqueued.
 *             dspark_last_error() gives a message (per host thread).
 *   Data.     Problems with the data itself (NaN rows, bad draws, ...) are
 *             reported per row / per request in device status arrays using
 *             the DSPARK_ST_* codes below.  Every output of a row or request
 *             with a nonzero status is zero (token 0, confidence 0.0,
 *             counts 0, sparse length 0, accept length 0, bonus 0) [C 6.3].
 *   Empty.    A call with no rows (n_rows == 0, or no requests) checks its
 *             scalar arguments and enqueues nothing; its array pointers may
 *             then be NULL.
 *   Threads.  The library is stateless and reentrant, except for the one
 *             allocation-free entry point, whose device scratch is shared.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSPARK_ABI_VERSION 2
#define DSPARK_MASS (1u << 24)   /* M, total count of a q row [Q] */
#define DSPARK_N_DRAFT 5         /* draft rows per request [C 2] */
#define DSPARK_N_TARGET 6        /* anchor + 5 target rows per request [A] */
#define DSPARK_K_MAX 1024        /* largest sparse top-k this build supports */
#define DSPARK_V_MAX (1 << 20)   /* largest vocabulary accepted */

/* host return codes */
#define DSPARK_SUCCESS 0
#define DSPARK_EINVAL (-1)       /* bad value, size, NULL pointer or mode */
#define DSPARK_EALIGN (-2)       /* row pointer or row stride not 16-byte aligned */
#define DSPARK_EWORKSPACE (-3)   /* workspace smaller than dspark_workspace_bytes() */
#define DSPARK_EHIP (-4)         /* the HIP runtime refused a launch */

/* device status codes (per row, per request) */
#define DSPARK_ST_OK 0
#define DSPARK_ST_ROW_NAN 1            /* a NaN logit or weight [Q] */
#define DSPARK_ST_ROW_POSINF 2         /* a +inf logit or weight [Q] */
#define DSPARK_ST_ROW_ZERO_MASS 3      /* every logit -inf / every weight 0 [Q] */
#define DSPARK_ST_DRAW_RANGE 4         /* a draw >= 2^24 [Q] */
#define DSPARK_ST_ALLOC_INCONSISTENT 5 /* remaining outside [0, #{r>0}] or sum != M [Q] */
#define DSPARK_ST_TARGET_INVALID 6     /* a target row of the request is invalid */
#define DSPARK_ST_DRAFT_INVALID 7      /* a valid draft row carries a token outside [0, V) */
#define DSPARK_ST_BAD_WEIGHT 8         /* weights-only entry: weight < 0 or > 1 */
#define DSPARK_ST_BAD_TOPK 9           /* topk[r] outside [0, min(k_max, V)] */
/* receiver-side refusals of a q row in the wire form [Q, "Versioned v2
 * message design"]; a row breaking several rules gets the smallest code */
#define DSPARK_ST_Q_BAD_LEN 10         /* sparse length outside [0, topk[r]] */
#define DSPARK_ST_Q_BAD_ID 11          /* sparse id outside [0, V) */
#define DSPARK_ST_Q_UNSORTED 12        /* sparse ids not strictly ascending (duplicates included) */
#define DSPARK_ST_Q_NONFINITE 13       /* a NaN or infinite value */
#define DSPARK_ST_Q_NEGATIVE 14        /* a value with the sign bit set (-0.0 included) */
#define DSPARK_ST_Q_NOT_DYADIC 15      /* value * 2^24 is not an integer */
#define DSPARK_ST_Q_PADDING 16         /* dense padding past V that is not +0.0 */
#define DSPARK_ST_Q_MASS 17            /* a value above 1, or counts not summing to M */
#define DSPARK_ST_Q_TOKEN 18           /* proposed token outside [0, V) or with q = 0 */

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;
typedef enum { DSPARK_GREEDY = 0, DSPARK_SAMPLED = 1 } dspark_mode;

/* A batch of V-wide logit rows (final logits: temperature and any bias are
 * applied upstream [Q]).  data: device pointer to row 0, float32 or bf16
 * (dtype); n_rows >= 0; 1 <= vocab <= DSPARK_V_MAX; row_stride >= vocab. */
typedef struct {
  const void* data;
  int32_t dtype;
  int32_t reserved;
  int64_t n_rows;
  int64_t vocab;
  int64_t row_stride;
} dspark_rows;

/* Storage for the dyadic24 q of n_rows rows [Q; layouts: "Size and
 * critical path"].  topk: device int32[n_rows]; topk[r] == 0 makes row r
 * dense, 1 <= topk[r] <= min(k_max, V) makes it sparse top-k; topk == NULL
 * makes every row dense.  k_max: 0..DSPARK_K_MAX, the row length of the
 * sparse arrays.
 *   dense:  uint32[n_rows][vocab] counts c_v (sum M); written only for dense
 *           rows; q(v) = c_v / 2^24.  May be NULL if no row is dense.
 *   sp_ids: int32[n_rows][k_max] support token ids, ascending, positive
 *           counts only; sp_cnt: uint32[n_rows][k_max] their counts;
 *   sp_len: int32[n_rows] number of entries written (0 for dense rows and
 *           failed rows).  May all be NULL if no row is sparse.          */
typedef struct {
  const int32_t* topk;
  int32_t k_max;
  int32_t reserved;
  uint32_t* dense;
  int32_t* sp_ids;
  uint32_t* sp_cnt;
  int32_t* sp_len;
} dspark_q;

/* Greedy proposal of every draft row [C 2]: argmax[r] = lowest index of the
 * row maximum (IEEE compare, -0 == +0); conf[r] = 1 / sum_v exp(x_v - max)
 * (softmax probability of the argmax, float32, within 1e-6 relative);
 * row_status[r] = OK / ROW_NAN / ROW_POSINF / ROW_ZERO_MASS (NaN is checked
 * first, then +inf, then all -inf).  Outputs are int32/float/int32[n_rows]. */
int dspark_propose(const dspark_rows* draft, int32_t* argmax, float* conf, int32_t* row_status,
                   void* ws, size_t ws_bytes, void* stream);

/* dyadic24-standard-v1 counts of every draft row [Q] ("allocate integer
 * counts"; this call does not allocate memory):
 *   support: all tokens (dense) or the top-k by (logit desc, id asc);
 *   m = row max; d_v = RN32(x_v - m); w_v = RN32(exp(d_v)) correctly rounded
 *   (-inf -> 0); S = sum_support w_v exactly; S64 = RN64(S);
 *   p_v = RN64(w_v / S64); y_v = p_v * 2^24; c_v = floor(y_v), r_v = y_v - c_v;
 *   remaining = M - sum c_v must satisfy 0 <= remaining <= #{r_v > 0};
 *   the `remaining` largest r_v (ties to the lowest id) get +1; sum c_v == M.
 * row_status[r] as in dspark_propose plus ALLOC_INCONSISTENT and BAD_TOPK. */
int dspark_q_alloc(const dspark_rows* draft, const dspark_q* q, int32_t* row_status, void* ws,
                   size_t ws_bytes, void* stream);

/* Integer categorical sampling [Q]: for row r and draw j, tokens[r][j] = the
 * first token (ascending id over the row's support) whose inclusive
 * cumulative count is strictly greater than draws[r][j].  draws: uint32
 * [n_rows][draws_per_row]; tokens: int32 same shape.  row_status is in/out:
 * rows that enter nonzero keep their status and get tokens 0; a draw
 * >= 2^24 sets DRAW_RANGE; counts that do not sum to M set
 * ALLOC_INCONSISTENT; either zeroes every token of the row.  Reads q->topk,
 * q->dense, q->sp_* as written by dspark_q_alloc. */
int dspark_sample(const dspark_q* q, int64_t n_rows, int64_t vocab, const uint32_t* draws,
                  int64_t draws_per_row, int32_t* tokens, int32_t* row_status, void* stream);

/* Greedy verification [A; C 2 anchor-as-first] of n_requests requests.
 * target: 6 rows per request (row i predicts draft position i; row 5 gives
 * only the bonus).  draft_tokens: int32[n_requests][5]; draft_status:
 * int32[n_requests][5] or NULL (all valid).  Outputs: target_argmax and
 * target_status int32[n_requests][6]; accept_len, bonus, req_status
 * int32[n_requests].  accept_len = number of leading positions whose draft
 * row is valid and whose token equals the target argmax (0..5); bonus =
 * target argmax at position accept_len.  Any invalid target row ->
 * TARGET_INVALID; a valid draft row with a token outside [0, V) ->
 * DRAFT_INVALID; both give accept_len = bonus = 0. */
int dspark_verify_greedy(const dspark_rows* target, const int32_t* draft_tokens,
                         const int32_t* draft_status, int64_t n_requests, int32_t* target_argmax,
                         int32_t* target_status, int32_t* accept_len, int32_t* bonus,
                         int32_t* req_status, void* ws, size_t ws_bytes, void* stream);

/* Stochastic verification [A, "State and sampling contracts": every target
 * row draws its own token from the target distribution with independent
 * noise; proposals are accepted while they match those draws, up to the
 * first mismatch].  The target distribution of a row is the full p at T = 1
 * [Q, "Distribution contract and precision": rounding to dyadic counts
 * changes the proposal only, not the legal target]: p_v = A_v / A with the
 * exact integers A_v = w_v 2^149 of the weights w_v = RN32(exp(RN32(x_v - m)))
 * and A = sum_v A_v.  Row i of request r takes the first token v (ascending
 * id) whose cumulative weight C_v satisfies C_v > floor(u A / 2^64), u =
 * target_draws[r][i] (uniform 64-bit; every value is valid).
 * target_draws: uint64[n_requests][6].  target_sample, target_status:
 * int32[n_requests][6] (a refused row: its status and token 0).
 * accept_len, bonus, req_status: int32[n_requests], with the rules of
 * dspark_verify_greedy applied to the drawn target tokens (bonus = the
 * target's draw at position accept_len).  Every target row is read once
 * (bf16 rows up to 131072 ids) or three times (float32 rows, longer rows). */
int dspark_verify_stochastic(const dspark_rows* target, const int32_t* draft_tokens,
                             const int32_t* draft_status, int64_t n_requests, const uint64_t* target_draws,
                             int32_t* target_sample, int32_t* target_status, int32_t* accept_len, int32_t* bonus,
                             int32_t* req_status, void* stream);

/* Probability-ratio verification with the dyadic q and full-vocabulary
 * residual sampling [Q, "Distribution contract and precision", last
 * paragraph: ratio tests and residual sampling use the full target p at
 * T = 1 and the defined q; "Sparse support and vocabulary-sharded TP2
 * follow-up": max(p - q, 0) for every token, including tokens outside a
 * sparse q's support; "Versioned v2 message design": zero q at the proposed
 * token is refused, acceptance and correction draws are separate].  p is the
 * distribution of dspark_verify_stochastic; q(v) = c_v / 2^24 from draft_q
 * (the draft rows' counts as dspark_q_alloc / dspark_fused write them, 5
 * rows per request).  Per request, at fixed depth five:
 *   - every draft row with status OK (draft_status int32[n][5], or NULL =
 *     all OK) must carry a token in [0, V) with q(token) > 0, else
 *     DRAFT_INVALID;
 *   - positions i = 0..4 in order read target row i (refused ->
 *     TARGET_INVALID); a draft row that failed ends the request with a draw
 *     from p_i; otherwise the proposal x is accepted when
 *     u_i c_x A < A_x 2^88 (U = u_i / 2^64 < p_i(x) / q_i(x), u_i =
 *     accept_draws[r][i]); on rejection the request ends with a draw from the
 *     residual, weights max(2^24 A_v - c_v A, 0), by the rule of
 *     dspark_verify_stochastic with u = final_draws[r];
 *   - after five acceptances, the bonus is drawn from p_5 with final_draws[r].
 * Target rows after the one that ends a request are not read.  Outputs
 * (int32[n_requests]): accept_len (0..5 committed proposals), token (the
 * correction or bonus token), req_status (OK, DRAFT_INVALID, TARGET_INVALID,
 * or ALLOC_INCONSISTENT for a zero residual, which needs counts that do not
 * sum to 2^24).  accept_draws: uint64[n_requests][5]; final_draws:
 * uint64[n_requests].  Six launches of n_requests workgroups; the outputs
 * carry the state between them, so they must not alias the inputs. */
int dspark_verify_ratio(const dspark_rows* target, const int32_t* draft_tokens, const int32_t* draft_status,
                        const dspark_q* draft_q, int64_t n_requests, const uint64_t* accept_draws,
                        const uint64_t* final_draws, int32_t* accept_len, int32_t* token, int32_t* req_status,
                        void* stream);

/* The whole step in one call: propose + (optional) q + (optional) sample on
 * the 5R draft rows, argmax on the 6R target rows, and greedy verification.
 * mode GREEDY verifies the argmax tokens, SAMPLED the sampled tokens (then q,
 * draws and sample are required).  q == NULL skips q; draws/sample == NULL
 * skip sampling (GREEDY only).  draws: uint32[5R], one per draft row. Output
 * shapes as in the single-stage calls; row_status covers the draft rows. */
int dspark_fused(const dspark_rows* draft, const dspark_rows* target, int32_t mode,
                 const dspark_q* q, const uint32_t* draws, int32_t* argmax, float* conf,
                 int32_t* sample, int32_t* row_status, int32_t* target_argmax,
                 int32_t* target_status, int32_t* accept_len, int32_t* bonus, int32_t* req_status,
                 void* ws, size_t ws_bytes, void* stream);

/* q rows in the wire form [Q, "Distribution contract and precision"]: each
 * value is c_v / 2^24 as a little-endian binary32, exact for c_v <= 2^24.
 *   topk:   as in dspark_q (device int32[n_rows]; 0 = dense row, else a
 *           sparse row of at most topk[r] entries; NULL = every row dense).
 *   dense:  float[n_rows][dense_stride]; a dense row sends `padded` values
 *           (vocab <= padded <= dense_stride, padded <= DSPARK_V_MAX + 64):
 *           the vocabulary, then padding that must be +0.0.  16-byte
 *           aligned, dense_stride a multiple of 4.  May be NULL if no row is
 *           dense.
 *   sp_ids: int32[n_rows][k_max], sp_val: float[n_rows][k_max] and
 *   sp_len: int32[n_rows], the first sp_len[r] entries of row r.  May be
 *           NULL if no row is sparse.                                     */
typedef struct {
  const int32_t* topk;
  int32_t k_max;
  int32_t reserved;
  const float* dense;
  int64_t padded;
  int64_t dense_stride;
  const int32_t* sp_ids;
  const float* sp_val;
  const int32_t* sp_len;
} dspark_q_wire;

/* Wire encoding of counts [Q]: values[i] = counts[i] / 2^24 as binary32
 * (the conversion rounds to nearest even, so counts above 2^24, which no
 * valid q holds, are not exact).  counts: uint32[n], values: float[n]
 * (device; may be the same memory).  Covers dense rows (n = rows * V) and
 * sparse count arrays alike; sparse ids travel unchanged. */
int dspark_q_encode(const uint32_t* counts, int64_t n, float* values, void* stream);

/* Receiver-side check of n_rows wire q rows [Q, "Versioned v2 message
 * design"; totals with 64-bit integers, no renormalisation, "Distribution
 * contract and precision"].  row_status[r] (int32[n_rows], required) gets
 * OK or the smallest DSPARK_ST_Q_* code (or BAD_TOPK for a bad topk[r] or a
 * dense row without dense storage) among the rules the row breaks.
 * tokens: int32[n_rows] proposed tokens, or NULL to skip that rule.
 * Recovered counts (optional): dense_counts uint32[n_rows][vocab] for dense
 * rows, sp_counts uint32[n_rows][k_max] for sparse rows (count of entry i at
 * i, zeros past sp_len[r]); a refused row's counts are all zero. */
int dspark_q_validate(const dspark_q_wire* q, int64_t n_rows, int64_t vocab, const int32_t* tokens,
                      uint32_t* dense_counts, uint32_t* sp_counts, int32_t* row_status, void* stream);

/* Margin of every row [C 6.3, the HAS_MARGIN reply field: top1 - top2 of
 * the logits, finite and >= 0; failed entries carry 0].  margin: float
 * [n_rows].  top2 is the second value in sorted order (a repeated maximum
 * gives 0); the binary32 difference m1 - m2, with a zero as +0.0; the
 * largest finite binary32 when no second finite logit exists or the
 * difference overflows; 0 for a row with a NaN, a +inf or only -inf.  One
 * extra read of the rows (the fused step does not compute it). */
int dspark_margin(const dspark_rows* rows, float* margin, void* stream);

/* Vocabulary-sharded propose, emulated on one GPU [Q, "Sparse support and
 * vocabulary-sharded TP2 follow-up"]: each row is cut into n_shards
 * contiguous shards (ids [g V / n_shards, (g + 1) V / n_shards)), each
 * handled by its own workgroup as a rank would; shard maxima are merged by
 * (value desc, id asc), the shards' exact integer weight sums are added and
 * rounded once.  Outputs (n_rows each; s64 and conf may be NULL): argmax,
 * s64 = RN64 of the exact sum of RN32(exp(RN32(x - max))), conf =
 * RN32(1 / s64), row_status (OK, ROW_NAN, ROW_POSINF, ROW_ZERO_MASS; a
 * refused row has argmax 0, s64 0, conf 0).  Every output is the same for
 * every n_shards in [1, min(64, vocab)].  ws: device scratch of at least
 * 48 * n_rows * n_shards bytes, 16-byte aligned (the shard results that
 * ranks would exchange). */
int dspark_sharded_propose(const dspark_rows* rows, int32_t n_shards, int32_t* argmax, double* s64, float* conf,
                           int32_t* row_status, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as dspark_sharded_propose, with the shard results kept in a fixed
 * device array inside the library (DSPARK_NOALLOC_SCRATCH_BYTES per GPU,
 * held until the process ends) instead of a caller workspace.  Nothing is
 * allocated.  Limit: n_rows * n_shards <= DSPARK_NOALLOC_ROW_SHARDS; a larger
 * call returns DSPARK_EWORKSPACE and enqueues nothing.  The array of the
 * current device is used (the stream must belong to that device); its
 * address is looked up on the first call on each device.  Every call on one
 * device shares that array: calls that overlap in time on one device race,
 * so the caller serialises them (one stream, or events). */
#define DSPARK_NOALLOC_SCRATCH_BYTES (1u << 22)
#define DSPARK_NOALLOC_ROW_SHARDS 87381 /* DSPARK_NOALLOC_SCRATCH_BYTES / 48 */
int dspark_sharded_propose_noalloc(const dspark_rows* rows, int32_t n_shards, int32_t* argmax, double* s64,
                                   float* conf, int32_t* row_status, void* stream);

/* Vocabulary-sharded q, emulated on one GPU [Q, "Sparse support and
 * vocabulary-sharded TP2 follow-up"]: the q of every row, and its sample, as
 * n_shards ranks holding contiguous shards (ids [g V / n_shards,
 * (g + 1) V / n_shards)) would compute them, with the values they would
 * exchange passed through ws:
 *   dense rows  - shard maxima and exact shard sums merged (every shard then
 *                 holds m and S64); each shard's floors and remainder keys;
 *                 remaining = M - the all-reduced floor sum; the bin of the
 *                 keys' top 11 bits where the `remaining` largest keys end,
 *                 from an all-reduced histogram; the ids inside that bin
 *                 gathered to the row's leader, which gives the bin's
 *                 tickets to its largest keys, ties to the lowest global id
 *                 across shards ("coordinate remaining tickets globally");
 *   sparse rows - each shard's local top-k (at most k candidates) merged by
 *                 (logit desc, global id asc) into the exact global top-k,
 *                 the counts allocated on that support;
 *   sample      - the draw (uint32, < 2^24) picks the shard whose
 *                 cumulative count mass first exceeds it, then the token in
 *                 that shard.
 * q (storage, topk, k_max), draws, argmax, sample and row_status as in
 * dspark_q_alloc / dspark_fused (draws and sample: both NULL or both
 * given).  Every output equals dspark_q_alloc's and the unsharded sample
 * for every n_shards in [1, min(64, V)].  Sparse rows need
 * n_shards * k_max <= 4096.  ws: at least dspark_sharded_q_workspace()
 * bytes (about 17 KB per row and shard and 8 KB per row, plus 8 B per
 * candidate slot of a sparse row), 256-byte aligned. */
size_t dspark_sharded_q_workspace(int64_t n_rows, int32_t n_shards, int32_t k_max);
int dspark_sharded_q(const dspark_rows* rows, int32_t n_shards, const dspark_q* q, const uint32_t* draws,
                     int32_t* argmax, int32_t* sample, int32_t* row_status, void* ws, size_t ws_bytes,
                     void* stream);

/* Test entry: the dense allocation steps of dspark_q_alloc applied to
 * caller-given float32 weights (normalised weights in [0, 1]), so that the
 * consistency assertions can be reached with constructed inputs.
 * w: float[n_rows] rows of n (stride elements apart); counts: uint32
 * [n_rows][n] (dense, stride n); row_status: ROW_NAN, ROW_POSINF,
 * BAD_WEIGHT, ROW_ZERO_MASS or ALLOC_INCONSISTENT on failure. */
int dspark_q_alloc_weights(const float* w, int64_t n_rows, int64_t n, int64_t stride,
                           uint32_t* counts, int32_t* row_status, void* ws, size_t ws_bytes,
                           void* stream);

/* Test entry: the library's weight function w = RN32(exp(d)) applied to n
 * float32 values d <= 0 (or -inf).  Used to check it exhaustively. */
int dspark_cr_expf(const float* d, float* w, int64_t n, void* stream);

/* Workspace bytes an entry point can use (op: 0 propose, 1 q_alloc, 2
 * sample, 3 verify, 4 fused, 5 q_alloc_weights; n_rows = draft rows).  No
 * entry point needs one (ws may be NULL with ws_bytes 0).  dspark_q_alloc
 * and dspark_fused use a workspace of at least this size, 256-byte aligned,
 * to run each dense-q draft row that is streamed from memory (float32
 * rows, bf16 rows above 131072 ids) through the split pipeline: the row's
 * vocabulary shards (min(64, 2048 / rows) of them, at least one), each a
 * workgroup per pass, merged as dspark_sharded_q merges them -- which fills
 * the chip when there are few rows and is faster than one workgroup per row
 * at every batch size; the results are the same either way.  It returns 0
 * where splitting does not apply (other ops, no draft rows). */
size_t dspark_workspace_bytes(int32_t op, int64_t n_rows, int64_t vocab, int32_t k_max);

const char* dspark_q_semantic_id(void); /* "dyadic24-standard-v1" [Q] */
const char* dspark_status_name(int32_t code);
const char* dspark_last_error(void);
int32_t dspark_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSPARK_H */
