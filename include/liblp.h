/*
 * liblp: deterministic, batch-invariant selected-token logprobs and the
 * three-way logprob comparison, for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every pointer argument is device memory owned by the caller unless
 * stated otherwise; the library allocates nothing and keeps no global state,
 * so calls on different streams may run concurrently. Calls enqueue work on
 * `stream` and return at once; results are valid once the stream has reached
 * them. Argument errors are returned synchronously before anything is
 * enqueued. No C++ exception crosses this interface.
 *
 * Sources (page titles as published):
 *   [AMD]  "Debugging Logprob Mismatches in LLM Reinforcement Learning"
 *   [vLLM] "Fault localization and mismatch bisect" (train-inference-
 *          consistency guide)
 *   [TII]  "Rollout-Training Mismatch in LLM RL"
 *   [RLK]  "Training and rollout stop disagreeing: vime and RL-Kernel hold
 *          logprobs bitwise identical for 200 steps on AMD MI300X"
 *   [VeX]  "Diagnosing Training Inference Mismatch in LLM Reinforcement
 *          Learning"
 */
#ifndef LIBLP_H
#define LIBLP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LP_OK = 0,
  LP_EINVAL = 1,       /* an argument is invalid; nothing was enqueued        */
  LP_EUNSUPPORTED = 2, /* valid, but a shape/alignment the library does not
                          handle; nothing was enqueued                        */
  LP_EHIP = 3          /* a HIP runtime call or kernel launch failed          */
} lp_status;

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* lp_status_string(lp_status status);

/* ------------------------------------------------------------------------
 * Selected-token logprob
 *
 * For every row t independently ([AMD] "Case 2: A and B Stay Close; C
 * Changes"; "How this differs from a real temperature mismatch"; "Collect
 * A/B and C"; [RLK] true vocabulary range):
 *
 *   z[t, v]       = sum_h hidden[t, h] * w[v, h]        (bf16 x bf16, fp32 acc.)
 *   s[t, v]       = z[t, v] / temperature               for v < V_true
 *   lse[t]        = log sum_{v < V_true} exp(s[t, v])    (natural log)
 *   logprob[t]    = s[t, target_ids[t]] - lse[t]         (nats, fp32)
 *
 * Rows are assumed already aligned with the tokens they predict (the
 * prediction after position j scores token j + 1, [AMD] "Align Each Score
 * With the Token It Predicts"); the binding's align() helper performs that
 * shift. Full logits are never written to memory.
 *
 * Determinism and batch invariance: each row's outputs are a fixed function
 * of that row's hidden vector, its target id, w, V_true and temperature. The
 * tile shape, the K (hidden) reduction order and the vocabulary merge order
 * are compile-time constants: they never depend on T, on the row's position
 * in the batch, on the other rows, on the stream or on the device occupancy.
 * There is no split-K and no floating-point atomic.
 *
 * Layout:
 *   hidden_bf16  [T, H] bf16, row stride ldh elements (ldh >= H, ldh % 8 == 0),
 *                16-byte aligned base.
 *   w_bf16       [V_rows, H] bf16, contiguous (row stride H), 16-byte aligned:
 *                the nn.Linear LM-head layout.
 *   target_ids   [T] int64.
 *   out_logprob  [T] fp32.
 *   out_lse      [T] fp32, may be NULL.
 *   bad_rows     one int32, may be NULL: the library ADDS the number of rows
 *                whose target id lies outside [0, V_true); the caller sets
 *                it to 0 beforehand. Such rows get logprob = NaN.
 *   workspace    at least lp_score_workspace_bytes(T, H, V_rows, V_true)
 *                bytes, 256-byte aligned; contents on entry are ignored.
 *
 * Errors: LP_EINVAL for T < 0, H < 1, V_rows < 1, V_true outside
 * [1, V_rows], ldh < H, a temperature that is not finite and > 0, a NULL
 * required pointer, or a workspace that is too small or misaligned.
 * LP_EUNSUPPORTED for H % 64 != 0, ldh % 8 != 0 or misaligned hidden/w; for
 * sizes whose dispatches would exceed 2^32 - 1 work-items (more than
 * 16 777 215 tiles of 352 x 256, or T above 268 435 455); and for
 * strides the kernels' 32-bit buffer addressing cannot span: 255 * ldh * 2 +
 * 2 * H or 352 * 2 * H above 0x7FFFFFF0 bytes (at H = 64 the largest
 * accepted ldh is 4 210 744; the largest accepted H is 3 050 368).
 * T == 0 is a no-op returning LP_OK.
 * ------------------------------------------------------------------------ */
size_t lp_score_workspace_bytes(int64_t T, int64_t H, int64_t V_rows,
                                int64_t V_true);

lp_status lp_score(const void* hidden_bf16, int64_t ldh, const void* w_bf16,
                   const int64_t* target_ids, int64_t T, int64_t H,
                   int64_t V_rows, int64_t V_true, float temperature,
                   float* out_logprob, float* out_lse, int32_t* bad_rows,
                   void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * lp_score without a caller workspace
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * call as lp_score, minus workspace and workspace_bytes, with the same
 * kernels and bit-identical outputs; the workspace is a device array of
 * LP_NOALLOC_SCRATCH_BYTES inside the library (one per device, held until
 * the process ends; its address is looked up once per device). No
 * allocation of any kind happens in the call.
 *
 * Limit: the workspace lp_score would need, lp_score_workspace_bytes(T, H,
 * V_rows, V_true), must fit LP_NOALLOC_SCRATCH_BYTES (32 MiB): at V_true =
 * 151 936, up to 9 697 rows. Larger calls return LP_EUNSUPPORTED before
 * anything is enqueued.
 *
 * Concurrency: every call on one device uses that device's one array, so
 * calls that overlap on a device (different streams, different threads)
 * race; order them (one stream, or events). The array keeps the last call's
 * contents, which no call reads before writing.
 *
 * Errors: as for lp_score (argument errors first), then LP_EUNSUPPORTED for
 * the scratch limit, LP_EHIP if the stream's device or the array's address
 * cannot be determined.
 * ------------------------------------------------------------------------ */
#define LP_NOALLOC_SCRATCH_BYTES (32u << 20)

lp_status lp_score_noalloc(const void* hidden_bf16, int64_t ldh,
                           const void* w_bf16, const int64_t* target_ids,
                           int64_t T, int64_t H, int64_t V_rows,
                           int64_t V_true, float temperature,
                           float* out_logprob, float* out_lse,
                           int32_t* bad_rows, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Selected-token logprob with the row's entropy and argmax
 *
 * The same call as lp_score, also returning per row the entropy of the
 * scored distribution and its most likely token, from the same fused pass
 * (the logits still never reach memory):
 *
 *   entropy[t] = -sum_{v < V_true} p[t, v] ln p[t, v],   p = softmax(s[t, :])
 *              = lse[t] - sum_v p[t, v] s[t, v]            (nats, fp32)
 *   argmax[t]  = the lowest v < V_true with z[t, v] = max_{v' < V_true} z[t, v']
 *                over the fp32 logits as this library computes them (int64)
 *
 * Sources: the trainer's scoring step that the AMD blog's Case 2 inspects
 * computes log probs and entropy together ([AMD] "Case 2: A and B Stay Close;
 * C Changes"); the full-vocabulary argmax is reported apart from the token
 * metrics ([vLLM] "Metric measurement basis"), and a top-1 token flip
 * between two scorings -- argmax differs for the same row -- is one of the
 * indicators [VeX] lists (result 1 and its list of practical indicators).
 * Two argmax arrays are compared as integers.
 *
 * out_logprob and out_lse hold exactly the bits lp_score writes for the same
 * arguments. The batch-invariance guarantee of lp_score covers entropy and
 * argmax too. Ties between logits that compare equal after the temperature
 * scale go to the lower index. Workspace: lp_score_stats_workspace_bytes (it
 * is larger than lp_score's). out_entropy [T] fp32 and out_argmax [T] int64
 * are required; every other argument, layout and error is as for lp_score.
 * ------------------------------------------------------------------------ */
size_t lp_score_stats_workspace_bytes(int64_t T, int64_t H, int64_t V_rows,
                                      int64_t V_true);

lp_status lp_score_stats(const void* hidden_bf16, int64_t ldh,
                         const void* w_bf16, const int64_t* target_ids,
                         int64_t T, int64_t H, int64_t V_rows, int64_t V_true,
                         float temperature, float* out_logprob, float* out_lse,
                         float* out_entropy, int64_t* out_argmax,
                         int32_t* bad_rows, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Scoring with options: lp_score_ex
 *
 * flags (bitwise or):
 *   LP_SCORE_STATS        also write out_entropy and out_argmax, exactly as
 *                         lp_score_stats (both then required)
 *   LP_SCORE_BF16_LOGITS  round every fp32-accumulated logit to bf16 (round
 *                         to nearest even) before the temperature and the
 *                         log-softmax, which stay fp32: the score a trainer
 *                         gets when its LM head stores logits in the model's
 *                         bf16 and only the final log-softmax is cast to fp32
 *                         ([AMD] "Collect A/B and C", notes on the trainer's
 *                         extraction: the fp32 cast applies to the final
 *                         log-softmax, upstream computation keeps its own
 *                         precision; [vLLM] "Metric measurement basis":
 *                         align the logits' precision before comparing).
 * flags = 0 is lp_score and flags = LP_SCORE_STATS is lp_score_stats, bit
 * for bit. Workspace: lp_score_ex_workspace_bytes(T, H, V_rows, V_true,
 * flags) (0 for invalid arguments). Errors as for lp_score, plus LP_EINVAL
 * for unknown flag bits.
 * ------------------------------------------------------------------------ */
#define LP_SCORE_STATS 1u
#define LP_SCORE_BF16_LOGITS 2u

size_t lp_score_ex_workspace_bytes(int64_t T, int64_t H, int64_t V_rows,
                                   int64_t V_true, uint32_t flags);

lp_status lp_score_ex(const void* hidden_bf16, int64_t ldh, const void* w_bf16,
                      const int64_t* target_ids, int64_t T, int64_t H,
                      int64_t V_rows, int64_t V_true, float temperature,
                      uint32_t flags, float* out_logprob, float* out_lse,
                      float* out_entropy, int64_t* out_argmax,
                      int32_t* bad_rows, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Three-way comparison of generation (A), replay (B) and trainer (C) scores
 *
 * [AMD] "One Response, Three Scores", "Check Whether the Pattern Extends",
 * Case 1's compare(); [vLLM] "Per-sequence observation patterns", "Metric
 * measurement basis", "Compare per-token logprobs"; [TII] sec. 2.1 (TIS);
 * [VeX] sec. 3 "How TIS takes effect" (token and sequence TIS).
 *
 * Pairs, in this order: p = 0: (A, B); p = 1: (B, C); p = 2: (A, C), written
 * (left, right). Per pair and per sequence n, over the ACTIVE tokens
 * (mask != 0) i_0 < i_1 < ... with active rank k:
 *
 *   valid        number of active tokens
 *   mismatch     active tokens whose fp32 bit patterns differ (+0.0 and -0.0
 *                differ, identical NaN bits do not). With atol >= 0, a token
 *                whose bits differ counts as equal when |left - right| <= atol.
 *   first_div    smallest active rank k that mismatches, -1 if none
 *   longest_run  longest run of consecutive active tokens that mismatch;
 *                inactive positions neither extend nor break a run
 *   nonfinite    active tokens whose left or right score is not finite; these
 *                take part in mismatch/first_div/longest_run only
 *   k3_nonfinite tokens whose k3 term overflows; left out of sum_k3
 *   delta_i      (double)left - (double)right; d_i = -delta_i
 *   max_abs      max |delta_i| (0 if none)          -- exact
 *   sum_abs      sum |delta_i|;  sum_signed = sum delta_i;  sum_d = sum d_i
 *   sum_k3       sum (expm1(d_i) - d_i)             (Schulman k3, never clipped)
 *   sum_tok_tis  sum min(exp(d_i), tis_clip)        (token TIS weights)
 *   seq_tis      min(exp(sum_d), tis_clip)          (sequence TIS weight)
 *
 * Integer fields and max_abs are exact. The fp64 sums are taken in a fixed
 * order, so they are bitwise reproducible run to run and independent of N.
 * sum_abs, sum_signed, sum_d and seq_tis are fp64 from the fp64 differences
 * (the library's tests hold them to 1e-9 relative of the exactly rounded
 * sums). Precision of the k3 and TIS terms:
 *   - |d_i| < 0.5: k3 = d^2 g(d) in fp32, with d the fp32 difference
 *     right - left (within an ulp of d_i) and g(d) = sum_k d^k / (k + 2)!
 *     by a degree-5 polynomial fitted on [-0.5, 0.5] (2.5e-8 relative, so
 *     no cancellation); the terms of each group of four consecutive
 *     positions are added in fp32 and the group sums in fp64. When
 *     tis_clip > e^0.5 (no such token reaches the cap), these tokens' share
 *     of sum_tok_tis is their count + their fp64 sum of d + their k3 sum
 *     (e^d = 1 + d + k3); otherwise each weight min(1 + d + k3, tis_clip) is
 *     rounded to fp32 and summed like k3.
 *   - |d_i| >= 0.5: both from one fp64 exponential, k3 = (e^d - 1) - d and
 *     min(e^d, tis_clip), summed in fp64.
 * sum_k3 and sum_tok_tis agree with the exactly rounded sums to about 1e-7
 * relative (the library's tests hold them to 1e-6). The per-token k3 and TIS
 * outputs carry the same per-term precision (fp32 weights 1 + d + k3 below
 * 0.5).
 *
 * Layout:
 *   gen_A, replay_B, train_C  [N, L] fp32, row stride ld elements (ld >= L).
 *   mask                      [N, L] uint8, same row stride ld.
 *   out                       [N][3] lp_seq_stats, sequence-major: out[3 n + p]
 *                             is pair p (0: (A,B), 1: (B,C), 2: (A,C)) of
 *                             sequence n. Device memory, 8-byte aligned.
 *   per_token                 NULL, or [3 pairs][3][N][L] fp32 contiguous with
 *                             values |delta|, k3, min(exp(d), tis_clip) for
 *                             active finite tokens, 0 for inactive tokens and
 *                             NaN for active non-finite ones.
 *
 * Errors: LP_EINVAL for N < 0, L < 0, ld < L, tis_clip not finite and > 0,
 * atol NaN, or a NULL required pointer; LP_EUNSUPPORTED for L above
 * INT32_MAX or N above 22 369 621 (one 192-thread workgroup per sequence in
 * one dispatch of at most 2^32 - 1 work-items). N == 0 or L == 0 is a no-op
 * (with L == 0 and N > 0 the stats are still written, all empty).
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t valid;
  int32_t mismatch;
  int32_t first_div;
  int32_t longest_run;
  int32_t nonfinite;
  int32_t k3_nonfinite;
  double max_abs;
  double sum_abs;
  double sum_signed;
  double sum_k3;
  double sum_d;
  double seq_tis;
  double sum_tok_tis;
} lp_seq_stats;

lp_status lp_compare(const float* gen_A, const float* replay_B,
                     const float* train_C, const uint8_t* mask, int64_t N,
                     int64_t L, int64_t ld, float tis_clip, float atol,
                     lp_seq_stats* out, float* per_token, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Quantiles of |Delta|: the rule used throughout
 *
 * p50, p95 and p99 follow numpy's default ("linear") quantile, the estimator
 * of the AMD blog's compare() (section "Case 1: A Changes; B and C Stay
 * Close", np.quantile(error, .95) and .99; the p95 / p99 row of "Check
 * Whether the Pattern Extends Across the Response" refers to it). Over n
 * counted values sorted ascending, x_0 <= ... <= x_{n-1}, and p = 0.5, 0.95,
 * 0.99: h = (n - 1) * p (one fp64 product); if h >= n - 1 the quantile is
 * x_{n-1}; otherwise, with j = floor(h), g = h - j, a = x_j, b = x_{j+1}:
 *   q = a + (b - a) * g          when g < 0.5
 *   q = b - (b - a) * (1 - g)    otherwise
 * each fp64 operation rounded on its own -- the bits np.quantile returns.
 * x_j and x_{j+1} are selected exactly (radix selection on the bit patterns
 * of |Delta|); 0 when n == 0.
 * ------------------------------------------------------------------------ */

/* ------------------------------------------------------------------------
 * Per-sequence quantiles: the blog's compare() applied to each record
 *
 * For each pair p (0: (A,B), 1: (B,C), 2: (A,C)) and sequence n, over the
 * sequence's counted tokens (active and both scores finite, Delta as for
 * lp_compare): out[(n * 3 + p) * 3 + j] = the quantile of |Delta| at
 * p = 0.5, 0.95, 0.99 for j = 0, 1, 2 (the rule above; 0 for a sequence
 * without counted tokens). Together with lp_compare's count, signed sum,
 * |Delta| sum and max_abs this is every field the AMD blog's compare()
 * returns, per record. With one counted token every quantile is its |Delta|.
 *
 * Layout and arguments as for lp_compare; out: [N][3][3] double in device
 * memory, 8-byte aligned. No workspace: each (sequence, pair) is selected
 * inside one workgroup. Exact and independent of N and of scheduling.
 *
 * Errors: LP_EINVAL for N < 0, L < 0, ld < L, a NULL or misaligned out, or
 * NULL inputs with N, L > 0; LP_EUNSUPPORTED for L above INT32_MAX or N
 * above 5 592 400 (three 256-thread workgroups per sequence, in groups of 8
 * sequences, in one dispatch of at most 2^32 - 1 work-items).
 * N == 0 does nothing; L == 0 writes zeros.
 * ------------------------------------------------------------------------ */
lp_status lp_compare_quantiles(const float* gen_A, const float* replay_B,
                               const float* train_C, const uint8_t* mask,
                               int64_t N, int64_t L, int64_t ld, double* out,
                               hipStream_t stream);

/* ------------------------------------------------------------------------
 * Batch tail statistics of the per-token differences
 *
 * For each pair (A,B), (B,C), (A,C) over the whole batch: the counted tokens
 * are the active ones whose two scores are finite, Delta as for lp_compare.
 * The batch pools every sequence's tokens: a run's distribution, which the
 * blog characterises from full response arrays.
 *
 *   count          number of counted tokens
 *   q50, q95, q99  quantiles of |Delta| over all counted tokens, by the rule
 *                  above (exact neighbours, fp64 interpolation); 0 when
 *                  count == 0
 *   max_abs        max |Delta| (0 when count == 0)
 *   max_seq, max_pos  sequence and column of the first counted token, in
 *                  row-major order, with |Delta| = max_abs (-1 when none)
 *   sum_abs        sum |Delta|                  (logprob_mae = sum_abs / count)
 *   sum_prob_abs   sum |exp(left) - exp(right)| (probability_mae numerator)
 *
 * [vLLM] "Metric measurement basis" (logprob_mae with its p95, max and
 * position; probability_mae); [VeX] section 5, practical indicators (p50 /
 * p95 / p99 / max of abs(delta_logprob)); [AMD] "Check Whether the Pattern
 * Extends Across the Response" (p95, p99, maximum, error by position).
 *
 * pos_abs_sum / pos_count (both NULL or both non-NULL): [3][L] arrays, pair-
 * major; for column i, the sum of |Delta| over the sequences whose token i
 * is counted, and how many are -- the error-by-position profile.
 *
 * Integer results, max values and the quantiles' order statistics are
 * exact, and the quantiles are np.quantile's bits; the fp64 sums are taken
 * in a fixed order (bitwise reproducible run to run).
 *
 * Layout and arguments as for lp_compare; out is [3] lp_tail_stats in device
 * memory; workspace: lp_compare_tails_workspace_bytes(N, L) bytes, 256-byte
 * aligned, contents ignored. Errors: LP_EINVAL for N < 0, L < 0, ld < L, a
 * NULL out or workspace, only one of pos_abs_sum / pos_count given, NULL
 * inputs with N, L > 0, or a small or misaligned workspace; LP_EUNSUPPORTED
 * for L above INT32_MAX, N above 16 777 215 (one 256-thread workgroup per
 * sequence in one dispatch of at most 2^32 - 1 work-items) or N * L above
 * 2^32 - 1 (32-bit histogram counters). N == 0 or L == 0 writes the empty
 * statistics (and zero profiles).
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t count;
  double q50;
  double q95;
  double q99;
  double max_abs;
  int32_t max_seq;
  int32_t max_pos;
  double sum_abs;
  double sum_prob_abs;
} lp_tail_stats;

size_t lp_compare_tails_workspace_bytes(int64_t N, int64_t L);

lp_status lp_compare_tails(const float* gen_A, const float* replay_B,
                           const float* train_C, const uint8_t* mask,
                           int64_t N, int64_t L, int64_t ld,
                           lp_tail_stats* out, double* pos_abs_sum,
                           int32_t* pos_count, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Batch tail statistics with the worst tokens
 *
 * lp_compare_tails plus, per pair, the k counted tokens with the largest
 * |Delta|: worst is [3][k] lp_worst_token in device memory (pair-major),
 * row j of pair p the (j+1)-th largest, ordered by |Delta| descending and,
 * among equal |Delta|, by row-major position (sequence, then column); when
 * the pair counts fewer than k tokens the remaining rows are {0.0, -1, -1}.
 * [vLLM] "Metric measurement basis": where the largest errors sit, not only
 * their mean; [VeX] section 5: the tail of abs(delta_logprob).
 *
 * The k-th largest |Delta| is selected exactly like the quantiles; the rows
 * are exact (bit-for-bit |Delta|, and the positions).
 *
 * 0 <= k <= LP_WORST_MAX; k == 0 gives lp_compare_tails (worst may be
 * NULL). Workspace: lp_compare_tails_ex_workspace_bytes(N, L, k) bytes,
 * 256-byte aligned. Errors as for lp_compare_tails, plus LP_EINVAL for k
 * outside [0, LP_WORST_MAX] or a NULL worst with k > 0.
 * ------------------------------------------------------------------------ */
#define LP_WORST_MAX 4096

typedef struct {
  double abs_delta;   /* |Delta| of the token */
  int32_t seq;        /* its sequence, -1 for a fill row */
  int32_t pos;        /* its column, -1 for a fill row */
} lp_worst_token;

size_t lp_compare_tails_ex_workspace_bytes(int64_t N, int64_t L, int32_t k);

lp_status lp_compare_tails_ex(const float* gen_A, const float* replay_B,
                              const float* train_C, const uint8_t* mask,
                              int64_t N, int64_t L, int64_t ld, int32_t k,
                              lp_tail_stats* out, lp_worst_token* worst,
                              double* pos_abs_sum, int32_t* pos_count,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * Vocabulary-parallel scoring with a canonical chunking
 *
 * With the LM head split over vocabulary shards, the normaliser must still
 * be one sum over the whole true vocabulary ([AMD] "Collect A/B and C", the
 * trainer-extraction notes: a vocabulary-parallel implementation needs a
 * global normaliser across shards), and the cross-rank LSE merge must use a
 * fixed reduction order ([RLK] the strict path: true vocabulary range,
 * cross-rank LSE merge, fixed rank reduction order).
 *
 * lp_score merges its per-tile partials in LP_MERGE_SEGMENTS fixed segments
 * of the 352-row vocabulary tiles (segment g holds tiles [g P, (g + 1) P),
 * P = ceil(ceil(V_true / 352) / 16)), each folded in ascending tile order,
 * then folds the segments in order. A shard owns whole segments:
 * lp_vocab_shard_range gives rank r of n (1 <= n <= 16) the segments
 * [16 r / n, 16 (r + 1) / n) and the vocabulary rows [row_begin, row_end)
 * they cover (empty when the vocabulary has fewer tiles than that).
 *
 * lp_score_shard scores one shard: w_shard_bf16 is rows [row_begin,
 * row_end) of W, contiguous [row_end - row_begin, H] bf16; the other
 * arguments are lp_score's with V_true the WHOLE true vocabulary size. It
 * writes the records of its own segments into `partials`, a buffer of
 * lp_shard_partials_bytes(T, flags) bytes laid out [16][F][T] fp32 (F = 3:
 * max and sum of exp2 in log2 units and the target's scaled logit, 0 where
 * the target is not in the segment; F = 5 with LP_SCORE_STATS: also the entropy term
 * and the argmax row as int32 bits). A rank's segments are one contiguous
 * byte range, so the exchange is one all-gather of T F 4 16 / n bytes per
 * rank (equal blocks when n divides 16). Workspace:
 * lp_score_shard_workspace_bytes(T, V_true, n, r, flags), 256-byte aligned.
 * flags are lp_score_ex's (LP_SCORE_STATS, LP_SCORE_BF16_LOGITS).
 *
 * lp_merge_shards folds the 16 records of each row in segment order and
 * writes what lp_score_ex with the same flags writes.
 * The results are BITWISE equal to lp_score_ex on the whole W
 * for any n: the tiles, their K order, every fold and its order are the
 * same. A target outside [0, V_true) gives NaN and ++*bad_rows in the merge.
 *
 * Errors: LP_EINVAL for T < 0, H < 1, ldh < H, V_true < 1, n outside
 * [1, 16], rank outside [0, n), unknown flag bits, a bad temperature, NULL
 * required pointers (hidden and w_shard may be NULL for an empty shard), a
 * small or misaligned workspace or a misaligned partials buffer;
 * LP_EUNSUPPORTED as for lp_score. T == 0 does nothing.
 * ------------------------------------------------------------------------ */
#define LP_MERGE_SEGMENTS 16
#define LP_VOCAB_TILE_ROWS 352  /* vocabulary rows per tile (the chunking unit) */

typedef struct {
  int32_t seg_lo;     /* first merge segment of the shard */
  int32_t seg_hi;     /* one past its last */
  int64_t row_begin;  /* first vocabulary row of the shard */
  int64_t row_end;    /* one past its last (<= V_true) */
} lp_vocab_shard;

lp_status lp_vocab_shard_range(int64_t V_true, int32_t n_shards, int32_t rank,
                               lp_vocab_shard* out);

size_t lp_shard_partials_bytes(int64_t T, uint32_t flags);

size_t lp_score_shard_workspace_bytes(int64_t T, int64_t V_true,
                                      int32_t n_shards, int32_t rank,
                                      uint32_t flags);

lp_status lp_score_shard(const void* hidden_bf16, int64_t ldh,
                         const void* w_shard_bf16, const int64_t* target_ids,
                         int64_t T, int64_t H, int64_t V_true,
                         float temperature, int32_t n_shards, int32_t rank,
                         uint32_t flags, void* partials, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

lp_status lp_merge_shards(const void* partials, const int64_t* target_ids,
                          int64_t T, int64_t V_true, uint32_t flags,
                          float* out_logprob, float* out_lse,
                          float* out_entropy, int64_t* out_argmax,
                          int32_t* bad_rows, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Correction consumers: TIS / MIS token weights and sequence rejection
 *
 * For each sequence n and active token i with both scores finite, the
 * correction ratio is r = pi_train / pi_rollout, taken in the log domain as
 * d = fp64(train_lp) - fp64(rollout_lp) (one IEEE operation):
 *
 *   weight   = 0                 unless mis_log_lo <= d <= mis_log_hi
 *            = C                 if d >= log C                 (TIS cap)
 *            = fp32(exp(d))      otherwise
 *   and weight = 0 on masked and non-finite tokens and in rejected
 *   sequences.
 *   stat     = sum over the counted tokens of K(r): K1 = -log r = -d,
 *              K3 = r - 1 - log r = expm1(d) - d (fp64; an overflowing
 *              term makes stat +inf); 0 with LP_REJECT_NONE
 *   accepted = reject_lo <= stat <= reject_hi
 *
 * ["Rollout-Training Mismatch in LLM RL"] section 2.1, Eq. (2) and the TIS /
 * MIS definitions after Eq. (3): w_TIS = min(w, C), w_MIS = w 1[l <= w <= u]
 * (here l = exp(mis_log_lo), u = exp(mis_log_hi); both may be combined);
 * [VeX] result 5 and the discussion of how TIS works: r_corr is the old
 * trainer over the rollout probability, token TIS clamps exp(log r) at C,
 * sequence rejection filters by sum_t K1(r_t) or sum_t K3(r_t), padding
 * tokens weigh 0.
 *
 * Arguments: rollout_lp, train_lp fp32 and mask uint8, [N, L] with row
 * stride ld (as for lp_compare); tis_clip C > 0 (+inf: no cap); the MIS
 * interval on log r (-inf / +inf: no bound); reject_kind LP_REJECT_NONE,
 * LP_REJECT_K1 or LP_REJECT_K3 and the accepted range of stat (-inf / +inf:
 * no bound). weights: [N, L] fp32 contiguous, or NULL for the statistics
 * only; out: [N] lp_corr_seq. Device memory owned by the caller; async on
 * `stream`.
 *
 * kept counts the counted tokens inside the interval whether or not the
 * sequence is accepted; capped those of them at the cap; sum_weight the
 * written weights (0 for a rejected sequence). Counts, accepted and the
 * interval / cap decisions are exact; stat and sum_weight are fp64 sums in a
 * fixed order (bitwise reproducible, independent of N).
 *
 * Errors: LP_EINVAL for N < 0, L < 0, ld < L, C <= 0 or NaN, a NaN or
 * inverted interval or accepted range, an unknown reject_kind, a NULL out,
 * or NULL inputs with N, L > 0; LP_EUNSUPPORTED for L above INT32_MAX or N
 * above 16 777 215 (one 256-thread workgroup per sequence in one dispatch).
 * N == 0 does nothing.
 * ------------------------------------------------------------------------ */
#define LP_REJECT_NONE 0
#define LP_REJECT_K1 1
#define LP_REJECT_K3 3

typedef struct {
  int32_t valid;      /* active tokens */
  int32_t nonfinite;  /* active tokens with a non-finite score (weight 0) */
  int32_t kept;       /* counted tokens inside the MIS interval */
  int32_t capped;     /* kept tokens whose weight is the cap C */
  int32_t accepted;   /* 1: the sequence is kept; 0: rejected */
  int32_t reserved;   /* 0 */
  double stat;        /* sum of K1 or K3 over the counted tokens */
  double sum_weight;  /* sum of the written weights */
} lp_corr_seq;

lp_status lp_correct(const float* rollout_lp, const float* train_lp,
                     const uint8_t* mask, int64_t N, int64_t L, int64_t ld,
                     double tis_clip, double mis_log_lo, double mis_log_hi,
                     int32_t reject_kind, double reject_lo, double reject_hi,
                     float* weights, lp_corr_seq* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBLP_H */
