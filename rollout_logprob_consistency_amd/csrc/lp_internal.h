// Internal launch interface between the C-ABI host code and the kernels.
// Not installed; the public interface is include/liblp.h.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "liblp.h"

namespace lp {

// Fixed tile geometry of the selected-token logprob. These never depend on
// the number of rows: every row is reduced over H and over the vocabulary in
// the same order whatever batch it is scored in.
constexpr int kTileV = 352;   // vocabulary rows per workgroup tile
constexpr int kTileT = 256;   // token rows per workgroup tile
constexpr int kTileK = 64;    // hidden elements per LDS stage
// Batches of at most this many rows take the streaming kernel (one wave per
// 128-row half of a vocabulary tile x 32 or 64 tokens, the same per-row
// arithmetic), which streams W at HBM rate instead of computing 256-token
// tiles that are mostly padding.
constexpr int kSkinnyMaxT = 64;
constexpr int kScoreTileThreads = 256;  // threads of a tile workgroup

struct ScoreArgs {
  const uint16_t* x;      // [T, ldh] bf16 bits
  const uint16_t* w;      // [V_rows, H] bf16 bits
  const int64_t* ids;     // [T]
  int64_t ldh;
  int32_t T, H, V_rows, V_true;
  int32_t v_base;         // vocabulary index of W row 0 (0 unless a shard)
  bool bf16_logits;       // round the fp32 logits to bf16 before the scale
  int32_t n_vt, n_tt;     // vocabulary / token tile counts
  float scale2;           // log2(e) / temperature
  float* part_m;          // [n_vt][T]  per-tile max (log2 units)
  float* part_s;          // [n_vt][T]  per-tile sum of exp2(s - max)
  float* tval;            // [T]        target logit (log2 units)
  float* out_lp;          // [T]
  float* out_lse;         // [T] or null
  int32_t* bad_rows;      // or null
  // Entropy / argmax outputs (lp_score_stats); null for lp_score.
  float* part_q;          // [rows][T]  per-partial sum 2^d d (log2 units)
  int32_t* part_i;        // [rows][T]  per-partial argmax (vocabulary row)
  float* out_ent;         // [T] entropy, nats
  int64_t* out_argmax;    // [T]
};

// Workspace layout inside the caller's buffer (offsets in bytes, 256-aligned).
// With stats, two more planes follow for the entropy term and the argmax.
struct ScoreWorkspace {
  size_t off_m, off_s, off_t, off_q, off_i, total;
};
ScoreWorkspace score_workspace_layout(int64_t T, int64_t V_true, bool stats);

hipError_t launch_score(const ScoreArgs& a, hipStream_t stream);

// Fixed merge segments of the vocabulary tiles; a vocabulary shard owns whole
// segments.
constexpr int kMergeSegs = 16;
static_assert(kMergeSegs == LP_MERGE_SEGMENTS, "the segment count is part of the C ABI");
static_assert(kTileV == LP_VOCAB_TILE_ROWS, "the tile height is part of the C ABI");
int merge_segment_tiles(int64_t V_true);  // tiles per segment

struct ShardArgs {
  int32_t seg_lo, n_seg;  // this shard's first segment and segment count
  int32_t per;            // vocabulary tiles per segment
  int32_t n_vt_glob;      // vocabulary tiles over the whole true range
  int32_t tile_base;      // tile index of this shard's first row
  int32_t V_true_glob;
  int32_t F;              // planes per segment record: 3, or 5 with stats
  float* out;             // [kMergeSegs][F][T] segment records
};
// ScoreArgs describe the shard's own rows (W = the shard, V_rows = V_true =
// its row count, v_base = its first row); the merge takes the whole range.
hipError_t launch_score_shard(const ScoreArgs& a, const ShardArgs& s, hipStream_t stream);
hipError_t launch_merge_shards(const ScoreArgs& a, const ShardArgs& s, hipStream_t stream);

// Row-parallel launches: one workgroup per sequence (three for the
// per-sequence quantiles), of these many threads. A dispatch holds at most
// 2^32 - 1 work-items, which bounds the sequences of one call.
constexpr int kCompareThreads = 192;
constexpr int kRowThreads = 256;  // correction, batch tails, per-sequence quantiles
constexpr int64_t kMaxDispatchItems = 0xFFFFFFFFll;

struct CompareArgs {
  const float* A;
  const float* B;
  const float* C;
  const uint8_t* mask;
  int64_t N, L, ld;
  double tis_clip;
  double log_clip;        // log(tis_clip)
  double atol;            // < 0: bitwise mode
  bool vec;               // rows 16-byte aligned (A, B, C) and 4-byte aligned (mask)
  lp_seq_stats* out;      // [N][3]: pair p of sequence n at 3 n + p
  float* per_token;       // [3][3][N][L] or null
};

hipError_t launch_compare(const CompareArgs& a, hipStream_t stream);

struct CorrectArgs {
  const float* rollout;   // [N, ld] log pi_rollout of the sampled tokens
  const float* train;     // [N, ld] log pi_train (old trainer) of the same tokens
  const uint8_t* mask;    // [N, ld]
  int64_t N, L, ld;
  int32_t kind;           // LP_REJECT_NONE / _K1 / _K3
  double cap, log_cap;    // TIS cap C and log C (log C = +inf: no cap)
  double log_lo, log_hi;  // MIS interval on log r
  double rej_lo, rej_hi;  // accepted range of the sequence statistic
  bool vec;               // rows 16-byte aligned and ld % 4 == 0
  float* weights;         // [N, L] or null
  lp_corr_seq* out;       // [N]
};

hipError_t launch_correct(const CorrectArgs& a, hipStream_t stream);

// Quantiles p = 0.5, 0.95, 0.99 of n >= 1 values by numpy's default
// ("linear") rule -- the estimator of the AMD blog's compare() (section
// "Case 1: A Changes; B and C Stay Close", np.quantile at its defaults).
// With h = (n - 1) p (one fp64 product) the result lies between the order
// statistics of 1-based ranks floor(h) + 1 and floor(h) + 2, or is the
// largest value when h >= n - 1.
__host__ __device__ inline double quantile_prob(int q) {
  return q == 0 ? 0.5 : (q == 1 ? 0.95 : 0.99);
}

__host__ __device__ inline void quantile_ranks(int64_t n, double p, int64_t* lo, int64_t* hi) {
  const double h = (double)(n - 1) * p;
  if (h >= (double)(n - 1)) {
    *lo = *hi = n;
    return;
  }
  const int64_t j = (int64_t)floor(h);
  *lo = j + 1;
  *hi = j + 2;
}

// The quantile from those two order statistics a <= b: the line between
// them at the fraction g = h - floor(h), taken from a when g < 1/2 and from
// b otherwise; each fp64 operation is rounded on its own (no contraction).
__host__ __device__ inline double quantile_lerp(int64_t n, double p, double a, double b) {
#pragma clang fp contract(off)
  const double h = (double)(n - 1) * p;
  if (h >= (double)(n - 1)) return b;
  const double g = h - floor(h);
  const double diff = b - a;
  return g < 0.5 ? a + diff * g : b - diff * (1.0 - g);
}

// Keys of |delta|: the bit pattern of the fp64 |l - r| of two finite fp32
// scores. As non-negative doubles the keys order like unsigned integers. The
// difference is 0 or has an fp64 exponent in [874, 1152] (2^-149 <= |delta|
// < 2^130), so the top 16 bits (exponent and four mantissa bits) take 4 464
// values; with the key 0 as bucket 0 that is 4 465 buckets, monotone in the
// key.
constexpr uint32_t kKeyTop16Lo = 874u << 4;          // top 16 bits of 2^-149
constexpr uint32_t kKeyTop16Hi = (1152u << 4) | 15u;  // top 16 bits just below 2^130
constexpr int kKeyBuckets = (int)(kKeyTop16Hi - kKeyTop16Lo) + 2;  // 4 465

__device__ __forceinline__ uint32_t key_bucket(uint64_t k) {
  const uint32_t t = (uint32_t)(k >> 48);
  return k == 0 ? 0u : min(max(t, kKeyTop16Lo), kKeyTop16Hi) - kKeyTop16Lo + 1u;
}

// The top 16 bits of the keys in bucket b > 0.
__device__ __forceinline__ uint64_t bucket_top16(uint32_t b) {
  return (uint64_t)(b - 1u + kKeyTop16Lo);
}

// Buffer resource (raw, 32-bit data format) over `bytes` bytes from `base`;
// wave-uniform, so it stays in SGPRs. Reads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), 0,
      (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Number of lanes below this one whose bit is set in m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Wave-aggregated LDS histogram increment of bin b for the lanes with hit
// (every lane of the wave calls it): when every hitting lane has the bin of
// the wave's first lane (read with readfirstlane, no LDS round trip), one
// atomic adds them all -- the common case for runs of equal keys.
__device__ __forceinline__ void wave_hist_add(uint32_t* h, uint32_t b, bool hit, int lane) {
  const uint64_t hb = __ballot(hit);
  if (hb == 0) return;
  const uint32_t b0 = __builtin_amdgcn_readfirstlane(b);
  if (__ballot(hit && b != b0) == 0) {
    if (lane == __ffsll((long long)hb) - 1) atomicAdd(&h[b0], (uint32_t)__popcll(hb));
  } else if (hit) {
    atomicAdd(&h[b], 1u);
  }
}

// The same add into 16-bit counters packed two to a 32-bit word (bin b in
// the low half of word b / 2 for even b) unless kWide: for rows of at most
// 65 535 positions no bin can overflow, and the histogram takes half the LDS.
template <bool kWide>
__device__ __forceinline__ void hist16_add(uint32_t* h, uint32_t b, bool hit, int lane) {
  const uint64_t hb = __ballot(hit);
  if (hb == 0) return;
  const uint32_t b0 = __builtin_amdgcn_readfirstlane(b);
  uint32_t bin = b, inc = 1u;
  if (__ballot(hit && b != b0) == 0) {
    if (lane != __ffsll((long long)hb) - 1) return;
    bin = b0;
    inc = (uint32_t)__popcll(hb);
  } else if (!hit) {
    return;
  }
  if (kWide) atomicAdd(&h[bin], inc);
  else atomicAdd(&h[bin >> 1], inc << ((bin & 1u) << 4));
}

struct TailArgs {
  const float* A;
  const float* B;
  const float* C;
  const uint8_t* mask;
  int64_t N, L, ld;
  lp_tail_stats* out;     // [3]
  double* pos_sum;        // [3][L] or null
  int32_t* pos_count;     // [3][L] or null (null iff pos_sum is)
  void* workspace;
  bool vec;               // rows 16-byte aligned (A, B, C), mask 4-byte aligned, ld % 4 == 0
  int32_t worst_k;        // worst tokens per pair (0: none)
  lp_worst_token* worst;  // [3][worst_k]; null when worst_k == 0
};

size_t tails_workspace_bytes(int64_t N, int64_t L, int32_t k);
hipError_t launch_tails(const TailArgs& a, hipStream_t stream);

struct QuantArgs {
  const float* A;
  const float* B;
  const float* C;
  const uint8_t* mask;
  int64_t N, L, ld;
  bool vec;               // rows 16-byte aligned (A, B, C), mask 4-byte aligned, ld % 4 == 0
  double* out;            // [N][3][3]: sequence, pair, quantile
};

hipError_t launch_seq_quantiles(const QuantArgs& a, hipStream_t stream);

// e^x in fp64 for finite x (the comparison's rare tokens with |d| >= 0.5 and
// the tail statistics' probabilities). Cody-Waite reduction x = k ln2 + r
// with ln2 split into a 32-bit head (k * head is exact for |k| < 2^21) and a
// tail, |r| <= ln2 / 2; e^r by its Taylor series to degree 12 (truncation
// < 2e-16 relative); then the exact scaling by 2^k, which overflows to +inf
// and underflows to 0 as the true value does. x is clamped to [-800, 800]
// first, beyond which e^x is already inf or 0.
__device__ __forceinline__ double exp_f64(double x) {
  constexpr double kLog2e = 0x1.71547652b82fep+0;
  constexpr double kLn2Hi = 0x1.62e42feep-1;
  constexpr double kLn2Lo = 0x1.a39ef35793c76p-33;
  x = fmin(fmax(x, -800.0), 800.0);
  const double k = rint(x * kLog2e);
  const double r = fma(-k, kLn2Lo, fma(-k, kLn2Hi, x));
  double p = 1.0 / 479001600.0;  // 1/12!
  p = fma(p, r, 1.0 / 39916800.0);
  p = fma(p, r, 1.0 / 3628800.0);
  p = fma(p, r, 1.0 / 362880.0);
  p = fma(p, r, 1.0 / 40320.0);
  p = fma(p, r, 1.0 / 5040.0);
  p = fma(p, r, 1.0 / 720.0);
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, (int)k);
}

// ---- Cross-lane steps of the XOR butterflies, without the LDS crossbar
// (the comparison and correction kernels' reductions).
// Step m pairs lane l with lane l ^ m. Every step leaves both lanes of a pair
// with the same value, so after steps 1 and 2 a quad is uniform and the half-
// row mirror (lane 7 - l of its 8) reads what lane l ^ 4 holds; after step 4
// the row mirror (lane 15 - l) reads lane l ^ 8's value. Step 16 swaps the
// 16-lane halves of each 32 with ds_swizzle; after it each 32-lane half is
// uniform and step 32 reads lanes 0 and 32 (readlane: a wave-uniform value).
template <int kM>
__device__ __forceinline__ int xlane(int v) {
  // Every source lane of these patterns exists and every row and bank is
  // enabled, so no lane keeps an old value (mov_dpp: none is materialised).
  if constexpr (kM == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  else if constexpr (kM == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  else if constexpr (kM == 4) return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  else if constexpr (kM == 8) return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);  // row_mirror
  else return __builtin_amdgcn_ds_swizzle(v, 0x401F);  // kM == 16: bit mode, lane ^ 16
}

template <int kM>
__device__ __forceinline__ double xlane(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = xlane<kM>((int)(uint32_t)b), hi = xlane<kM>((int)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// The value of lane `l` once each 32-lane half is uniform.
__device__ __forceinline__ int lane_value(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ double lane_value(double v, int l) {
  const long long b = __double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum / maximum over the wave by the fixed XOR butterfly; every lane gets the
// value lane 0 forms, ((x_0 + x_1) + (x_2 + x_3)) + ... (fp64 addition is
// commutative, so both lanes of a step agree bitwise).
template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
  x += xlane<1>(x);
  x += xlane<2>(x);
  x += xlane<4>(x);
  x += xlane<8>(x);
  x += xlane<16>(x);
  return lane_value(x, 0) + lane_value(x, 32);
}

__device__ __forceinline__ double wave_max(double x) {
  x = fmax(x, xlane<1>(x));
  x = fmax(x, xlane<2>(x));
  x = fmax(x, xlane<4>(x));
  x = fmax(x, xlane<8>(x));
  x = fmax(x, xlane<16>(x));
  return fmax(lane_value(x, 0), lane_value(x, 32));
}

}  // namespace lp
