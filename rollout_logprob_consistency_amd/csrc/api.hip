// C-ABI entry points of liblp: argument validation, workspace layout, fixed
// launch geometry. Every check happens before anything is enqueued.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <limits>
#include <mutex>

#include "lp_internal.h"

namespace {

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

constexpr int64_t kI32Max = std::numeric_limits<int32_t>::max();

// The scoring kernels address a tile's rows through buffer resources with
// 32-bit byte offsets and a range of at most kSpanMax bytes from the tile's
// first row: a token tile reaches 255 rows of stride ldh plus one row of H
// elements, a vocabulary tile 352 rows of H. Larger strides would read rows
// past the range as zeros, so they are refused.
constexpr uint64_t kSpanMax = 0x7FFFFFF0ull;

bool spans_ok(int64_t ldh, int64_t H) {
  if (ldh < 1 || H < 1 || (uint64_t)ldh > kSpanMax || (uint64_t)H > kSpanMax) return false;
  return (uint64_t)(lp::kTileT - 1) * (uint64_t)ldh * 2 + (uint64_t)H * 2 <= kSpanMax &&
         (uint64_t)lp::kTileV * (uint64_t)H * 2 <= kSpanMax;
}
constexpr uint32_t kScoreFlags = LP_SCORE_STATS | LP_SCORE_BF16_LOGITS;

// The scoring dispatches fit 2^32 - 1 work-items: n_vt x n_tt tile
// workgroups, and the merge's workgroup of 64 x 16 threads per 64 rows.
bool score_grid_ok(int64_t T, int64_t n_vt, int64_t n_tt) {
  return n_vt * n_tt <= lp::kMaxDispatchItems / lp::kScoreTileThreads &&
         (T + 63) / 64 <= lp::kMaxDispatchItems / (64 * lp::kMergeSegs);
}

// Sequences whose workgroups (wg_per_row of `threads` each) fit one dispatch.
bool rows_fit(int64_t N, int64_t wg_per_row, int64_t threads) {
  return N <= lp::kMaxDispatchItems / (wg_per_row * threads);
}

// Canonical shard of the merge segments: rank r of n owns segments
// [16 r / n, 16 (r + 1) / n) and the vocabulary rows they cover.
lp_vocab_shard shard_of(int64_t V_true, int32_t n_shards, int32_t rank) {
  const int64_t rows_per_seg = (int64_t)lp::merge_segment_tiles(V_true) * lp::kTileV;
  lp_vocab_shard s;
  s.seg_lo = (int32_t)((int64_t)lp::kMergeSegs * rank / n_shards);
  s.seg_hi = (int32_t)((int64_t)lp::kMergeSegs * (rank + 1) / n_shards);
  s.row_begin = std::min<int64_t>(V_true, s.seg_lo * rows_per_seg);
  s.row_end = std::min<int64_t>(V_true, s.seg_hi * rows_per_seg);
  return s;
}

bool shard_args_ok(int64_t V_true, int32_t n_shards, int32_t rank) {
  return V_true >= 1 && V_true <= kI32Max && n_shards >= 1 && n_shards <= lp::kMergeSegs &&
         rank >= 0 && rank < n_shards;
}

}  // namespace

extern "C" {

lp_status lp_vocab_shard_range(int64_t V_true, int32_t n_shards, int32_t rank,
                               lp_vocab_shard* out) {
  if (!out || !shard_args_ok(V_true, n_shards, rank)) return LP_EINVAL;
  *out = shard_of(V_true, n_shards, rank);
  return LP_OK;
}

size_t lp_shard_partials_bytes(int64_t T, uint32_t flags) {
  if (T < 0 || T > kI32Max || (flags & ~kScoreFlags)) return 0;
  return (size_t)lp::kMergeSegs * ((flags & LP_SCORE_STATS) ? 5 : 3) * (size_t)T * sizeof(float);
}

size_t lp_score_shard_workspace_bytes(int64_t T, int64_t V_true, int32_t n_shards, int32_t rank,
                                      uint32_t flags) {
  if (T < 0 || T > kI32Max || !shard_args_ok(V_true, n_shards, rank) || (flags & ~kScoreFlags))
    return 0;
  const lp_vocab_shard sh = shard_of(V_true, n_shards, rank);
  const size_t total =
      lp::score_workspace_layout(T, sh.row_end - sh.row_begin, (flags & LP_SCORE_STATS) != 0).total;
  return total < 256 ? 256 : total;
}

lp_status lp_score_shard(const void* hidden_bf16, int64_t ldh, const void* w_shard_bf16,
                         const int64_t* target_ids, int64_t T, int64_t H, int64_t V_true,
                         float temperature, int32_t n_shards, int32_t rank, uint32_t flags,
                         void* partials, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (T < 0 || H < 1 || ldh < H || !shard_args_ok(V_true, n_shards, rank)) return LP_EINVAL;
  if (flags & ~kScoreFlags) return LP_EINVAL;
  const bool stats = (flags & LP_SCORE_STATS) != 0;
  if (!(isfinite(temperature) && temperature > 0.0f)) return LP_EINVAL;
  if (T == 0) return LP_OK;
  const lp_vocab_shard sh = shard_of(V_true, n_shards, rank);
  const int64_t rows = sh.row_end - sh.row_begin;
  if (!target_ids || !partials || !workspace) return LP_EINVAL;
  if (rows > 0 && (!hidden_bf16 || !w_shard_bf16)) return LP_EINVAL;
  const lp::ScoreWorkspace ws = lp::score_workspace_layout(T, rows, stats);
  if (workspace_bytes < ws.total || !aligned(workspace, 256) || !aligned(partials, 4))
    return LP_EINVAL;
  if (H % lp::kTileK != 0 || ldh % 8 != 0) return LP_EUNSUPPORTED;
  if (rows > 0 && (!aligned(hidden_bf16, 16) || !aligned(w_shard_bf16, 16)))
    return LP_EUNSUPPORTED;
  const int64_t n_vt = (rows + lp::kTileV - 1) / lp::kTileV;
  const int64_t n_tt = (T + lp::kTileT - 1) / lp::kTileT;
  if (T > kI32Max || H > kI32Max || !score_grid_ok(T, n_vt, n_tt) || !spans_ok(ldh, H))
    return LP_EUNSUPPORTED;

  lp::ScoreArgs a;
  a.x = static_cast<const uint16_t*>(hidden_bf16);
  a.w = static_cast<const uint16_t*>(w_shard_bf16);
  a.ids = target_ids;
  a.ldh = ldh;
  a.T = (int32_t)T;
  a.H = (int32_t)H;
  a.V_rows = (int32_t)rows;
  a.V_true = (int32_t)rows;
  a.v_base = (int32_t)sh.row_begin;
  a.bf16_logits = (flags & LP_SCORE_BF16_LOGITS) != 0;
  a.n_vt = (int32_t)n_vt;
  a.n_tt = (int32_t)n_tt;
  a.scale2 = (float)(1.4426950408889634 / (double)temperature);
  char* base = static_cast<char*>(workspace);
  a.part_m = reinterpret_cast<float*>(base + ws.off_m);
  a.part_s = reinterpret_cast<float*>(base + ws.off_s);
  a.tval = reinterpret_cast<float*>(base + ws.off_t);
  a.out_lp = nullptr;
  a.out_lse = nullptr;
  a.bad_rows = nullptr;
  a.part_q = stats ? reinterpret_cast<float*>(base + ws.off_q) : nullptr;
  a.part_i = stats ? reinterpret_cast<int32_t*>(base + ws.off_i) : nullptr;
  a.out_ent = nullptr;
  a.out_argmax = nullptr;

  lp::ShardArgs s;
  s.seg_lo = sh.seg_lo;
  s.n_seg = sh.seg_hi - sh.seg_lo;
  s.per = lp::merge_segment_tiles(V_true);
  s.n_vt_glob = (int32_t)((V_true + lp::kTileV - 1) / lp::kTileV);
  s.tile_base = (int32_t)(sh.row_begin / lp::kTileV);
  s.V_true_glob = (int32_t)V_true;
  s.F = stats ? 5 : 3;
  s.out = static_cast<float*>(partials);
  if (s.n_seg == 0) return LP_OK;
  return lp::launch_score_shard(a, s, stream) == hipSuccess ? LP_OK : LP_EHIP;
}

lp_status lp_merge_shards(const void* partials, const int64_t* target_ids, int64_t T,
                          int64_t V_true, uint32_t flags, float* out_logprob, float* out_lse,
                          float* out_entropy, int64_t* out_argmax, int32_t* bad_rows,
                          hipStream_t stream) {
  if (T < 0 || V_true < 1 || (flags & ~kScoreFlags)) return LP_EINVAL;
  const bool stats = (flags & LP_SCORE_STATS) != 0;
  if (T == 0) return LP_OK;
  if (!partials || !target_ids || !out_logprob || !aligned(partials, 4)) return LP_EINVAL;
  if (stats && (!out_entropy || !out_argmax)) return LP_EINVAL;
  if (T > kI32Max || V_true > kI32Max) return LP_EUNSUPPORTED;
  lp::ScoreArgs a = {};
  a.ids = target_ids;
  a.T = (int32_t)T;
  a.V_true = (int32_t)V_true;
  a.out_lp = out_logprob;
  a.out_lse = out_lse;
  a.bad_rows = bad_rows;
  a.out_ent = stats ? out_entropy : nullptr;
  a.out_argmax = stats ? out_argmax : nullptr;
  lp::ShardArgs s = {};
  s.per = lp::merge_segment_tiles(V_true);
  s.F = stats ? 5 : 3;
  s.out = static_cast<float*>(const_cast<void*>(partials));
  return lp::launch_merge_shards(a, s, stream) == hipSuccess ? LP_OK : LP_EHIP;
}

const char* lp_status_string(lp_status status) {
  switch (status) {
    case LP_OK: return "LP_OK: success";
    case LP_EINVAL: return "LP_EINVAL: invalid argument (nothing was enqueued)";
    case LP_EUNSUPPORTED:
      return "LP_EUNSUPPORTED: shape or alignment not supported (nothing was enqueued)";
    case LP_EHIP: return "LP_EHIP: HIP runtime or kernel launch failure";
  }
  return "unknown lp_status";
}

size_t lp_score_workspace_bytes(int64_t T, int64_t H, int64_t V_rows, int64_t V_true) {
  (void)H;
  if (T < 0 || V_rows < 1 || V_true < 1 || V_true > V_rows) return 0;
  return lp::score_workspace_layout(T, V_true, false).total;
}

size_t lp_score_stats_workspace_bytes(int64_t T, int64_t H, int64_t V_rows, int64_t V_true) {
  (void)H;
  if (T < 0 || V_rows < 1 || V_true < 1 || V_true > V_rows) return 0;
  return lp::score_workspace_layout(T, V_true, true).total;
}

}  // extern "C"

namespace {

// Shared body of lp_score and lp_score_stats (stats: entropy and argmax
// requested, both non-NULL).
lp_status score_impl(const void* hidden_bf16, int64_t ldh, const void* w_bf16,
                     const int64_t* target_ids, int64_t T, int64_t H, int64_t V_rows,
                     int64_t V_true, float temperature, float* out_logprob, float* out_lse,
                     float* out_entropy, int64_t* out_argmax, bool stats, bool bf16,
                     int32_t* bad_rows, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  if (T < 0 || H < 1 || V_rows < 1 || V_true < 1 || V_true > V_rows || ldh < H)
    return LP_EINVAL;
  if (!(isfinite(temperature) && temperature > 0.0f)) return LP_EINVAL;
  if (T == 0) return LP_OK;
  if (!hidden_bf16 || !w_bf16 || !target_ids || !out_logprob || !workspace) return LP_EINVAL;
  if (stats && (!out_entropy || !out_argmax)) return LP_EINVAL;
  const lp::ScoreWorkspace ws = lp::score_workspace_layout(T, V_true, stats);
  if (workspace_bytes < ws.total || !aligned(workspace, 256)) return LP_EINVAL;
  if (H % lp::kTileK != 0 || ldh % 8 != 0) return LP_EUNSUPPORTED;
  if (!aligned(hidden_bf16, 16) || !aligned(w_bf16, 16)) return LP_EUNSUPPORTED;
  const int64_t n_vt = (V_true + lp::kTileV - 1) / lp::kTileV;
  const int64_t n_tt = (T + lp::kTileT - 1) / lp::kTileT;
  if (T > kI32Max || H > kI32Max || V_rows > kI32Max || !score_grid_ok(T, n_vt, n_tt) ||
      !spans_ok(ldh, H))
    return LP_EUNSUPPORTED;

  lp::ScoreArgs a;
  a.x = static_cast<const uint16_t*>(hidden_bf16);
  a.w = static_cast<const uint16_t*>(w_bf16);
  a.ids = target_ids;
  a.ldh = ldh;
  a.T = (int32_t)T;
  a.H = (int32_t)H;
  a.V_rows = (int32_t)V_rows;
  a.V_true = (int32_t)V_true;
  a.v_base = 0;
  a.bf16_logits = bf16;
  a.n_vt = (int32_t)n_vt;
  a.n_tt = (int32_t)n_tt;
  a.scale2 = (float)(1.4426950408889634 / (double)temperature);
  char* base = static_cast<char*>(workspace);
  a.part_m = reinterpret_cast<float*>(base + ws.off_m);
  a.part_s = reinterpret_cast<float*>(base + ws.off_s);
  a.tval = reinterpret_cast<float*>(base + ws.off_t);
  a.out_lp = out_logprob;
  a.out_lse = out_lse;
  a.bad_rows = bad_rows;
  a.part_q = stats ? reinterpret_cast<float*>(base + ws.off_q) : nullptr;
  a.part_i = stats ? reinterpret_cast<int32_t*>(base + ws.off_i) : nullptr;
  a.out_ent = stats ? out_entropy : nullptr;
  a.out_argmax = stats ? out_argmax : nullptr;
  return lp::launch_score(a, stream) == hipSuccess ? LP_OK : LP_EHIP;
}

}  // namespace

extern "C" {

lp_status lp_score(const void* hidden_bf16, int64_t ldh, const void* w_bf16,
                   const int64_t* target_ids, int64_t T, int64_t H, int64_t V_rows,
                   int64_t V_true, float temperature, float* out_logprob, float* out_lse,
                   int32_t* bad_rows, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  return score_impl(hidden_bf16, ldh, w_bf16, target_ids, T, H, V_rows, V_true, temperature,
                    out_logprob, out_lse, nullptr, nullptr, false, false, bad_rows, workspace,
                    workspace_bytes, stream);
}

lp_status lp_score_stats(const void* hidden_bf16, int64_t ldh, const void* w_bf16,
                         const int64_t* target_ids, int64_t T, int64_t H, int64_t V_rows,
                         int64_t V_true, float temperature, float* out_logprob, float* out_lse,
                         float* out_entropy, int64_t* out_argmax, int32_t* bad_rows,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return score_impl(hidden_bf16, ldh, w_bf16, target_ids, T, H, V_rows, V_true, temperature,
                    out_logprob, out_lse, out_entropy, out_argmax, true, false, bad_rows,
                    workspace, workspace_bytes, stream);
}

size_t lp_score_ex_workspace_bytes(int64_t T, int64_t H, int64_t V_rows, int64_t V_true,
                                   uint32_t flags) {
  if (T < 0 || H < 1 || V_true < 1 || V_true > V_rows || (flags & ~kScoreFlags)) return 0;
  return lp::score_workspace_layout(T, V_true, (flags & LP_SCORE_STATS) != 0).total;
}

lp_status lp_score_ex(const void* hidden_bf16, int64_t ldh, const void* w_bf16,
                      const int64_t* target_ids, int64_t T, int64_t H, int64_t V_rows,
                      int64_t V_true, float temperature, uint32_t flags, float* out_logprob,
                      float* out_lse, float* out_entropy, int64_t* out_argmax,
                      int32_t* bad_rows, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (flags & ~kScoreFlags) return LP_EINVAL;
  const bool stats = (flags & LP_SCORE_STATS) != 0;
  return score_impl(hidden_bf16, ldh, w_bf16, target_ids, T, H, V_rows, V_true, temperature,
                    out_logprob, out_lse, stats ? out_entropy : nullptr,
                    stats ? out_argmax : nullptr, stats, (flags & LP_SCORE_BF16_LOGITS) != 0,
                    bad_rows, workspace, workspace_bytes, stream);
}

lp_status lp_compare(const float* gen_A, const float* replay_B, const float* train_C,
                     const uint8_t* mask, int64_t N, int64_t L, int64_t ld, float tis_clip,
                     float atol, lp_seq_stats* out, float* per_token, hipStream_t stream) {
  if (N < 0 || L < 0 || ld < L) return LP_EINVAL;
  if (!(isfinite(tis_clip) && tis_clip > 0.0f) || isnan(atol)) return LP_EINVAL;
  if (N == 0) return LP_OK;
  if (!out) return LP_EINVAL;
  if (L > 0 && (!gen_A || !replay_B || !train_C || !mask)) return LP_EINVAL;
  if (L > kI32Max || !rows_fit(N, 1, lp::kCompareThreads)) return LP_EUNSUPPORTED;
  lp::CompareArgs a;
  a.A = gen_A;
  a.B = replay_B;
  a.C = train_C;
  a.mask = mask;
  a.N = N;
  a.L = L;
  a.ld = ld;
  a.tis_clip = (double)tis_clip;
  a.log_clip = log((double)tis_clip);
  a.atol = atol < 0.0f ? -1.0 : (double)atol;
  a.out = out;
  a.per_token = per_token;
  a.vec = ld % 4 == 0 && aligned(gen_A, 16) && aligned(replay_B, 16) && aligned(train_C, 16) &&
          aligned(mask, 4);
  return lp::launch_compare(a, stream) == hipSuccess ? LP_OK : LP_EHIP;
}

lp_status lp_correct(const float* rollout_lp, const float* train_lp, const uint8_t* mask,
                     int64_t N, int64_t L, int64_t ld, double tis_clip, double mis_log_lo,
                     double mis_log_hi, int32_t reject_kind, double reject_lo, double reject_hi,
                     float* weights, lp_corr_seq* out, hipStream_t stream) {
  if (N < 0 || L < 0 || ld < L) return LP_EINVAL;
  if (isnan(tis_clip) || !(tis_clip > 0.0)) return LP_EINVAL;
  if (isnan(mis_log_lo) || isnan(mis_log_hi) || mis_log_lo > mis_log_hi) return LP_EINVAL;
  if (isnan(reject_lo) || isnan(reject_hi) || reject_lo > reject_hi) return LP_EINVAL;
  if (reject_kind != LP_REJECT_NONE && reject_kind != LP_REJECT_K1 &&
      reject_kind != LP_REJECT_K3)
    return LP_EINVAL;
  if (N == 0) return LP_OK;
  if (!out) return LP_EINVAL;
  if (L > 0 && (!rollout_lp || !train_lp || !mask)) return LP_EINVAL;
  if (L > kI32Max || !rows_fit(N, 1, lp::kRowThreads)) return LP_EUNSUPPORTED;
  lp::CorrectArgs a;
  a.rollout = rollout_lp;
  a.train = train_lp;
  a.mask = mask;
  a.N = N;
  a.L = L;
  a.ld = ld;
  a.kind = reject_kind;
  a.cap = tis_clip;
  a.log_cap = log(tis_clip);
  a.log_lo = mis_log_lo;
  a.log_hi = mis_log_hi;
  a.rej_lo = reject_lo;
  a.rej_hi = reject_hi;
  a.weights = weights;
  a.out = out;
  a.vec = ld % 4 == 0 && aligned(rollout_lp, 16) && aligned(train_lp, 16) && aligned(mask, 4) &&
          aligned(weights, 16);
  return lp::launch_correct(a, stream) == hipSuccess ? LP_OK : LP_EHIP;
}

lp_status lp_compare_quantiles(const float* gen_A, const float* replay_B, const float* train_C,
                               const uint8_t* mask, int64_t N, int64_t L, int64_t ld, double* out,
                               hipStream_t stream) {
  if (N < 0 || L < 0 || ld < L) return LP_EINVAL;
  if (N == 0) return LP_OK;
  if (!out || !aligned(out, 8)) return LP_EINVAL;
  if (L > 0 && (!gen_A || !replay_B || !train_C || !mask)) return LP_EINVAL;
  // Three workgroups per sequence, in groups of 8 sequences.
  if (L > kI32Max || !rows_fit((N + 7) / 8 * 8, 3, lp::kRowThreads)) return LP_EUNSUPPORTED;
  lp::QuantArgs a;
  a.A = gen_A;
  a.B = replay_B;
  a.C = train_C;
  a.mask = mask;
  a.N = N;
  a.L = L;
  a.ld = ld;
  a.vec = ld % 4 == 0 && aligned(gen_A, 16) && aligned(replay_B, 16) && aligned(train_C, 16) &&
          aligned(mask, 4);
  a.out = out;
  return lp::launch_seq_quantiles(a, stream) == hipSuccess ? LP_OK : LP_EHIP;
}

size_t lp_compare_tails_workspace_bytes(int64_t N, int64_t L) {
  return lp_compare_tails_ex_workspace_bytes(N, L, 0);
}

size_t lp_compare_tails_ex_workspace_bytes(int64_t N, int64_t L, int32_t k) {
  if (N < 0 || L < 0 || N > kI32Max || L > kI32Max || k < 0 || k > LP_WORST_MAX) return 0;
  return lp::tails_workspace_bytes(N, L, k);
}

lp_status lp_compare_tails(const float* gen_A, const float* replay_B, const float* train_C,
                           const uint8_t* mask, int64_t N, int64_t L, int64_t ld,
                           lp_tail_stats* out, double* pos_abs_sum, int32_t* pos_count,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return lp_compare_tails_ex(gen_A, replay_B, train_C, mask, N, L, ld, 0, out, nullptr,
                             pos_abs_sum, pos_count, workspace, workspace_bytes, stream);
}

lp_status lp_compare_tails_ex(const float* gen_A, const float* replay_B, const float* train_C,
                              const uint8_t* mask, int64_t N, int64_t L, int64_t ld, int32_t k,
                              lp_tail_stats* out, lp_worst_token* worst, double* pos_abs_sum,
                              int32_t* pos_count, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  if (N < 0 || L < 0 || ld < L) return LP_EINVAL;
  if (!out || !workspace) return LP_EINVAL;
  if (k < 0 || k > LP_WORST_MAX || (k > 0 && !worst)) return LP_EINVAL;
  if ((pos_abs_sum == nullptr) != (pos_count == nullptr)) return LP_EINVAL;
  if (N > 0 && L > 0 && (!gen_A || !replay_B || !train_C || !mask)) return LP_EINVAL;
  // One workgroup per sequence; 32-bit histogram counters (N L tokens at most).
  if (L > kI32Max || !rows_fit(N, 1, lp::kRowThreads) || N * L > lp::kMaxDispatchItems)
    return LP_EUNSUPPORTED;
  if (workspace_bytes < lp::tails_workspace_bytes(N, L, k) || !aligned(workspace, 256))
    return LP_EINVAL;
  if (k > 0 && !aligned(worst, 8)) return LP_EINVAL;
  lp::TailArgs a;
  a.A = gen_A;
  a.B = replay_B;
  a.C = train_C;
  a.mask = mask;
  a.N = N;
  a.L = L;
  a.ld = ld;
  a.out = out;
  a.pos_sum = pos_abs_sum;
  a.pos_count = pos_count;
  a.workspace = workspace;
  a.vec = ld % 4 == 0 && aligned(gen_A, 16) && aligned(replay_B, 16) && aligned(train_C, 16) &&
          aligned(mask, 4);
  a.worst_k = k;
  a.worst = worst;
  return lp::launch_tails(a, stream) == hipSuccess ? LP_OK : LP_EHIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// lp_score_noalloc: lp_score with its workspace in this library's own device
// memory, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace (per-tile partials and target logits, fully written by the
// scoring kernels before the merge reads them, so nothing needs clearing)
// lives in `scratch`, one copy per device for the life of the process. In
// host code `scratch` names a host-side stand-in, never the device memory:
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that address reaches a kernel. Calls
// that overlap on one device share the array and race; the caller orders
// them (one stream, or events).
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[LP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev`, looked up on first use.
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

lp_status lp_score_noalloc(const void* hidden_bf16, int64_t ldh, const void* w_bf16,
                           const int64_t* target_ids, int64_t T, int64_t H, int64_t V_rows,
                           int64_t V_true, float temperature, float* out_logprob,
                           float* out_lse, int32_t* bad_rows, hipStream_t stream) {
  // Argument errors first, exactly as lp_score reports them; then the
  // scratch limit; only then any HIP call.
  if (T < 0 || H < 1 || V_rows < 1 || V_true < 1 || V_true > V_rows || ldh < H)
    return LP_EINVAL;
  if (!(isfinite(temperature) && temperature > 0.0f)) return LP_EINVAL;
  if (T == 0) return LP_OK;
  if (!hidden_bf16 || !w_bf16 || !target_ids || !out_logprob) return LP_EINVAL;
  if (lp::score_workspace_layout(T, V_true, false).total > (size_t)LP_NOALLOC_SCRATCH_BYTES)
    return LP_EUNSUPPORTED;
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess)
    return LP_EHIP;
  void* ws = nullptr;
  if (scratch_address(dev, &ws) != hipSuccess) return LP_EHIP;
  return score_impl(hidden_bf16, ldh, w_bf16, target_ids, T, H, V_rows, V_true, temperature,
                    out_logprob, out_lse, nullptr, nullptr, false, false, bad_rows, ws,
                    (size_t)LP_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
