// Batch tail statistics of the three-way comparison on gfx950
// (lp_compare_tails, lp_compare_tails_ex): per pair, p50 / p95 / p99 of
// |delta| by numpy's default (linear) quantile rule, the worst token, the
// k worst tokens, probability and logprob error sums and the per-position
// error profile. The per-sequence comparison itself is in compare.hip.
#include <math.h>

#include <type_traits>

#include "lp_internal.h"

namespace lp {

// ---------------------------------------------------------------------------
// Batch tail statistics of |delta| per pair (lp_compare_tails): the p50 / p95
// / p99 / max of abs(delta_logprob) that "Diagnosing Training Inference
// Mismatch in LLM Reinforcement Learning" (section 5, practical indicators)
// asks to record, and the logprob_mae / probability_mae numerators with the
// worst token's position of "Fault localization and mismatch bisect" ("Metric
// measurement basis"), plus the error-by-position profile.
//
// Quantiles follow numpy's default ("linear") rule, the estimator of the
// AMD blog's compare(): each lies between two neighbouring order statistics
// (quantile_ranks), which are selected exactly and interpolated in fp64
// (quantile_lerp). The order statistics are found by radix selection on the
// keys (the bit patterns of |delta|, which order like the values). A
// selection target is one rank of one pair: the two ranks of each quantile
// and, with worst tokens, the k-th largest. Targets of a pair whose known
// prefixes agree see the same tokens; the first of them (the "source") takes
// the histogram or the gather, and the others read it.
//  Pass 0  reads the batch once (one workgroup per sequence): the 4 465-bucket
//          histogram of the keys' top 16 bits per pair, and the per-sequence
//          sums and maxima. A one-workgroup select finds every target's
//          bucket and its rank inside it.
//  Pass 1  reads the batch again: each source histograms byte [47:40] of the
//          keys in its bucket and copies those keys into a list region of
//          the exact size (the bucket's count; the region is split by
//          histogram copy, so each sequence's workgroup appends to the part
//          that its copy counted). A source whose bucket holds at most 4 096
//          keys gathers them instead.
//  Pass 2 .. 6  select bytes [39:32] .. [7:0] from the lists (the batch, for
//          a source whose list did not fit the key buffer). Once a source's
//          prefix holds at most 4 096 keys it gathers them in the next pass
//          and leaves the passes.
//  Finish  one workgroup per gathering source selects its targets' remaining
//          bytes from the gathered keys in LDS.
// Every count is an integer, so the result does not depend on the order in
// which workgroups run or append. The sums and the first worst token are
// formed per sequence in a fixed order (pass 0) and reduced in a fixed tree;
// the position profile folds fixed chunks of sequences in order.
//
// Worst k tokens: the k-th largest key tau of a pair is selected like the
// quantiles; then every sequence counts its tokens above tau and equal to
// it, a scan turns the counts into offsets, and a second pass writes the
// tokens above tau and the first (in row-major order) of those equal to it
// as candidates; one workgroup per pair sorts its candidates (|delta|
// descending, then sequence and column ascending).
// ---------------------------------------------------------------------------
namespace {

// Targets per pair: the lower and upper neighbouring ranks of p50, p95 and
// p99 (targets 2q and 2q + 1) and, when worst tokens are asked for, the k-th
// largest (target 6). The kernels are instantiated for 6 and 7 (an idle
// seventh target would still cost every pass a little); the workspace always
// has room for 7.
constexpr int kMaxTP = 7;
constexpr int kWorstT = 6;  // index of the k-th-largest target within a pair
constexpr int kMaxTargets = 3 * kMaxTP;
constexpr int kTailThreads = kRowThreads;
constexpr int kTailChunks = 128;    // sequence chunks of the position profile
// Histogram copies: the workgroup of sequence n adds into copy n mod 8 (with
// workgroups dealt to the 8 XCDs in turn, each copy is one XCD's), so no
// counter takes atomics from more than N / 8 workgroups.
constexpr int kCopies = 8;
constexpr int kB16Pad = 4480;       // words per pass-0 pair histogram (>= kKeyBuckets)
constexpr int kHistStride = kMaxTargets * 256;  // words per byte-histogram copy
constexpr int kGather = 4096;       // keys a source gathers for the finish
constexpr int kLastPass = 6;        // pass p >= 1 selects key bits [55 - 8p : 48 - 8p]
// Atomic counters that many workgroups update sit 256 bytes apart, each in
// a cache line of its own.
constexpr int kCtrStride64 = 32;    // int64 counters
constexpr int kCtrStride32 = 64;    // uint32 counters
static_assert(kTailThreads == 256, "one byte-histogram bin per thread");
static_assert(kB16Pad >= kKeyBuckets && kB16Pad % 64 == 0, "pass-0 histogram rows");

__device__ __forceinline__ int pass_shift(int pass) { return 48 - 8 * pass; }

struct TailSel {
  uint64_t prefix;   // known top bits of the selected key (the key itself when done)
  int64_t rank;      // 1-based rank still wanted under that prefix; 0: done or none
  int32_t lreg;      // list region that holds its candidates (-1: none, read the batch)
  int32_t fin_src;   // source whose gathered keys finish it (-1: none)
  int32_t fin_bits;  // key bits below the prefix when it was gathered
  int32_t pad;
};

struct TailPart {    // one (sequence, pair), from pass 0
  double sum_abs, sum_prob;
  uint64_t max_key;  // bits of the largest |delta| (0 without tokens)
  int32_t max_pos;   // its first column, -1 without tokens
  int32_t count;
};

// x followed by y: sums added, counts added, the larger |delta| kept (equal
// maxima keep the lower column). Every operation is commutative, so the two
// lanes of a butterfly step get the same result.
__device__ __forceinline__ TailPart tail_part_combine(TailPart x, const TailPart& y) {
  x.sum_abs += y.sum_abs;
  x.sum_prob += y.sum_prob;
  x.count += y.count;
  if (y.max_pos >= 0 &&
      (x.max_pos < 0 || y.max_key > x.max_key || (y.max_key == x.max_key && y.max_pos < x.max_pos))) {
    x.max_key = y.max_key;
    x.max_pos = y.max_pos;
  }
  return x;
}

struct TailList {    // region of keys[] that a pass-0 source fills in pass 1
  int64_t off, len;
};

// What the next pass does, written by the select before it and read by the
// pass with a handful of independent loads, so that a pass with nothing to
// do exits after one.
struct TailPlan {
  uint64_t pre[kMaxTargets];  // each target's known prefix
  int32_t lsrc[kMaxTargets];  // the list region its source reads (-1: the batch)
  int8_t src[kMaxTargets];    // the target whose histogram target t reads
  uint32_t hist;              // sources that histogram this pass's byte
  uint32_t gath;              // sources that gather their keys in this pass
  uint32_t own;               // pass 1: sources that fill their list region
};

struct WorstCand {   // a worst-token candidate
  uint64_t key;      // bits of |delta|
  int32_t seq, pos;
};

struct TailWs {
  uint32_t* hist0;   // [kCopies][3][kB16Pad]
  uint32_t* hist;    // [kCopies][kMaxTargets][256], right after hist0
  TailSel* sel;      // [kMaxTargets]
  TailList* list;    // [kMaxTargets], by owning source
  TailPlan* plan;
  int64_t* fill;     // [kMaxTargets][kCopies][kCtrStride64] pass-1 write cursors
  uint32_t* gcnt;    // [kMaxTargets][kCtrStride32] gathered keys per source
  uint64_t* gbuf;    // [kMaxTargets][kGather]
  uint64_t* keys;    // [3][cap], one key buffer per pair
  int64_t cap;
  int64_t* count;    // [3]
  TailPart* part;    // [N][3]
  double* pos_part;  // [nch][3][L]
  int32_t* pos_cpart;
  int nch;
  int32_t k;         // worst tokens per pair (0: none)
  uint32_t* wcnt;    // [2][3][N] tokens above / equal to tau, per pair and sequence
  int64_t* woff;     // [2][3][N] their offsets (exclusive scan over sequences)
  WorstCand* cand;   // [3][k]
};

__host__ __device__ inline size_t tail_up(size_t x) { return (x + 255) & ~size_t(255); }

// Key buffer of a pair: a quarter of the positions. The sources of a pair
// sit in different buckets, so their lists are disjoint; a list that does
// not fit leaves its source reading the batch.
inline int64_t tail_key_cap(int64_t N, int64_t L) { return (N * L + 3) / 4; }

constexpr size_t kHist0Words = (size_t)kCopies * 3 * kB16Pad;
constexpr size_t kHistWords = (size_t)kCopies * kHistStride;
static_assert((kHist0Words * 4) % 256 == 0, "hist follows hist0 contiguously");

// One pass over the layout: with base == nullptr it only sizes it.
size_t tail_walk(char* p, int64_t N, int64_t L, int32_t k, TailWs* w) {
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* q = p ? p + o : nullptr;
    o = tail_up(o + bytes);
    return q;
  };
  TailWs x;
  x.hist0 = reinterpret_cast<uint32_t*>(take(kHist0Words * sizeof(uint32_t)));
  x.hist = reinterpret_cast<uint32_t*>(take(kHistWords * sizeof(uint32_t)));
  x.sel = reinterpret_cast<TailSel*>(take(kMaxTargets * sizeof(TailSel)));
  x.list = reinterpret_cast<TailList*>(take(kMaxTargets * sizeof(TailList)));
  x.plan = reinterpret_cast<TailPlan*>(take(sizeof(TailPlan)));
  x.fill = reinterpret_cast<int64_t*>(take((size_t)kMaxTargets * kCopies * kCtrStride64 * sizeof(int64_t)));
  x.gcnt = reinterpret_cast<uint32_t*>(take((size_t)kMaxTargets * kCtrStride32 * sizeof(uint32_t)));
  x.gbuf = reinterpret_cast<uint64_t*>(take((size_t)kMaxTargets * kGather * sizeof(uint64_t)));
  x.cap = tail_key_cap(N, L);
  x.keys = reinterpret_cast<uint64_t*>(take((size_t)3 * x.cap * sizeof(uint64_t)));
  x.count = reinterpret_cast<int64_t*>(take(3 * sizeof(int64_t)));
  x.part = reinterpret_cast<TailPart*>(take((size_t)N * 3 * sizeof(TailPart)));
  x.nch = (int)(N < kTailChunks ? (N < 1 ? 1 : N) : kTailChunks);
  x.pos_part = reinterpret_cast<double*>(take((size_t)x.nch * 3 * L * sizeof(double)));
  x.pos_cpart = reinterpret_cast<int32_t*>(take((size_t)x.nch * 3 * L * sizeof(int32_t)));
  x.k = k;
  x.wcnt = reinterpret_cast<uint32_t*>(take((size_t)(k > 0 ? 6 * N : 0) * sizeof(uint32_t)));
  x.woff = reinterpret_cast<int64_t*>(take((size_t)(k > 0 ? 6 * N : 0) * sizeof(int64_t)));
  x.cand = reinterpret_cast<WorstCand*>(take((size_t)(k > 0 ? 3 * k : 0) * sizeof(WorstCand)));
  if (w) *w = x;
  return o;
}

TailWs tail_layout(void* base, int64_t N, int64_t L, int32_t k) {
  TailWs w;
  tail_walk(static_cast<char*>(base), N, L, k, &w);
  return w;
}

size_t tail_bytes(int64_t N, int64_t L, int32_t k) { return tail_walk(nullptr, N, L, k, nullptr); }

// Left and right side of pair p among the three scores (A, B, C).
__device__ __forceinline__ int pair_left(int p) { return p == 1 ? 1 : 0; }
__device__ __forceinline__ int pair_right(int p) { return p == 0 ? 1 : 2; }

// Position profile, stage 1: each thread sums its column over chunk c's
// sequences (fixed chunks, sequences in ascending order); the final kernel
// folds the chunks in order. One column per thread: with 4-byte loads the
// launch has four times the waves of a 4-column form (16-byte loads), whose
// 1.5 waves per SIMD left the reads latency-bound (the call took 1.5 % longer);
// a column's sum is the same either way.
__device__ void tails_pos_chunk(const TailArgs& a, const TailWs& w, int64_t i0, int c) {
  if (i0 >= a.L) return;
  const int64_t per = (a.N + w.nch - 1) / w.nch;
  const int64_t lo = c * per, hi = min(a.N, lo + per);
  double s[3] = {};
  int32_t k[3] = {};
  // Four sequences' loads are issued together (all of them, masked or not).
  constexpr int kB = 4;
  for (int64_t n0 = lo; n0 < hi; n0 += kB) {
    float v[kB][3];
    bool act[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const bool in = n0 + b < hi;
      const int64_t o = (in ? n0 + b : lo) * a.ld + i0;
      act[b] = in && a.mask[o] != 0;
      v[b][0] = act[b] ? a.A[o] : 0.f;
      v[b][1] = act[b] ? a.B[o] : 0.f;
      v[b][2] = act[b] ? a.C[o] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      if (!act[b]) continue;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const float l = v[b][pair_left(p)], r = v[b][pair_right(p)];
        if (!__builtin_isfinite(l) || !__builtin_isfinite(r)) continue;
        s[p] += fabs((double)l - (double)r);
        k[p] += 1;
      }
    }
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    w.pos_part[((size_t)c * 3 + p) * a.L + i0] = s[p];
    w.pos_cpart[((size_t)c * 3 + p) * a.L + i0] = k[p];
  }
}

// Clears the histograms (every copy) and the gather counts, and resets the
// selection state; with the position profile asked for (pos true, grid
// ceil(L / 256) x chunks), workgroup (x, c) also forms stage 1 of the profile
// for columns [256 x, 256 (x + 1)) of chunk c.
constexpr int kInitBlocks = 64;

__global__ __launch_bounds__(kTailThreads) void tails_init_kernel(TailArgs a, TailWs w, bool pos) {
  uint4* z = reinterpret_cast<uint4*>(w.hist0);
  constexpr int64_t kVecs = (int64_t)(kHist0Words + kHistWords) / 4;
  const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  for (int64_t i = wg * kTailThreads + threadIdx.x; i < kVecs;
       i += (int64_t)gridDim.x * gridDim.y * kTailThreads)
    z[i] = make_uint4(0u, 0u, 0u, 0u);
  if (pos) tails_pos_chunk(a, w, (int64_t)blockIdx.x * kTailThreads + threadIdx.x, (int)blockIdx.y);
  if (wg != 0) return;
  const int t = threadIdx.x;
  if (t < kMaxTargets) {
    w.gcnt[t * kCtrStride32] = 0u;
    w.sel[t] = TailSel{0ull, 0, -1, -1, 0, 0};
    w.list[t] = TailList{0, 0};
  }
  if (t == 0) {
    w.plan->hist = 0u;
    w.plan->gath = 0u;
    w.plan->own = 0u;
  }
}

// Scores and mask of the four positions i .. i + 3 of row n (inactive past
// L); 16-byte loads on the vector path, element loads otherwise.
template <bool kVec>
__device__ __forceinline__ void tail_load4(const TailArgs& a, const float* const rows[3],
                                           const uint8_t* M, int64_t i, float v[4][3],
                                           bool act[4]) {
  if (kVec && i + 4 <= a.L) {
    const uint32_t mv = *reinterpret_cast<const uint32_t*>(M + i);
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const float4 f = *reinterpret_cast<const float4*>(rows[s] + i);
      v[0][s] = f.x;
      v[1][s] = f.y;
      v[2][s] = f.z;
      v[3][s] = f.w;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) act[k] = ((mv >> (8 * k)) & 255u) != 0;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      act[k] = i + k < a.L && M[i + k] != 0;
#pragma unroll
      for (int s = 0; s < 3; ++s) v[k][s] = act[k] ? rows[s][i + k] : 0.f;
    }
  }
}

// Counted flag and key of pair p at one position.
__device__ __forceinline__ bool tail_key(const float v[3], bool act, int p, uint64_t* key) {
  const float l = v[pair_left(p)], r = v[pair_right(p)];
  *key = (uint64_t)__double_as_longlong(fabs((double)l - (double)r));
  return act && __builtin_isfinite(l) && __builtin_isfinite(r);
}

// Pass 0's histogram increments are hist16_add: 32-bit counters, or (kWide
// false, rows of at most 65 535 positions) two 16-bit counters per word, so
// that the three pairs' histograms take 26.8 KB of LDS instead of 53.6 KB.

// Pass 0: the bucket histogram of every pair, and each sequence's sums and
// maximum, over one row per workgroup.
template <bool kVec, bool kWide>
__global__ __launch_bounds__(kTailThreads) void tails_p0_kernel(TailArgs a, TailWs w) {
  constexpr int kWords = kWide ? kKeyBuckets : (kKeyBuckets + 1) / 2;
  __shared__ uint32_t h[3 * kWords];
  __shared__ TailPart red[3][kTailThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < 3 * kWords; i += kTailThreads) h[i] = 0u;
  __syncthreads();

  const int64_t n = blockIdx.x;
  const float* const rows[3] = {a.A + n * a.ld, a.B + n * a.ld, a.C + n * a.ld};
  const uint8_t* M = a.mask + n * a.ld;
  TailPart mine[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) mine[p] = TailPart{0.0, 0.0, 0ull, -1, 0};
  // Groups of four consecutive positions 4 tid + 1024 k; the trip count is
  // the same for every thread, so every lane of a wave takes part in the
  // ballots (positions past L are inactive). Positions ascend within a
  // thread.
  constexpr int64_t kStep = 4 * kTailThreads;
  const int64_t Lw = (a.L + kStep - 1) / kStep * kStep;
  for (int64_t i0 = 4 * (int64_t)tid; i0 < Lw; i0 += kStep) {
    float vv[4][3];
    bool actv[4];
    tail_load4<kVec>(a, rows, M, i0, vv, actv);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float* v = vv[k];
      // e^A, e^B, e^C of an active token (0 if not finite). When every active
      // lane of the wave has bitwise equal B and A (or C and B), e^B (e^C) is
      // the exponential already formed (a uniform test).
      const bool act = actv[k];
      const bool ab = __float_as_uint(v[0]) == __float_as_uint(v[1]);
      const bool bc = __float_as_uint(v[1]) == __float_as_uint(v[2]);
      const bool same_ab = __ballot(act && !ab) == 0, same_bc = __ballot(act && !bc) == 0;
      double e[3];
      e[0] = act && __builtin_isfinite(v[0]) ? exp_f64((double)v[0]) : 0.0;
      if (same_ab) e[1] = e[0];
      else e[1] = act && __builtin_isfinite(v[1]) ? exp_f64((double)v[1]) : 0.0;
      if (same_bc) e[2] = e[1];
      else e[2] = act && __builtin_isfinite(v[2]) ? exp_f64((double)v[2]) : 0.0;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        uint64_t key;
        const bool ok = tail_key(v, actv[k], p, &key);
        hist16_add<kWide>(h + p * kWords, key_bucket(key), ok, lane);
        if (!ok) continue;
        TailPart& m = mine[p];
        m.sum_abs += __longlong_as_double((long long)key);
        m.sum_prob += fabs(e[pair_left(p)] - e[pair_right(p)]);
        if (m.max_pos < 0 || key > m.max_key) {  // positions ascend: the first one stays
          m.max_key = key;
          m.max_pos = (int32_t)(i0 + k);
        }
        m.count += 1;
      }
    }
  }
  __syncthreads();
  uint32_t* g = w.hist0 + (size_t)(n % kCopies) * 3 * kB16Pad;
  for (int i = tid; i < 3 * kWords; i += kTailThreads) {
    const uint32_t v = h[i];
    if (v == 0u) continue;
    const int p = i / kWords, wd = i - p * kWords;
    if (kWide) {
      atomicAdd(&g[p * kB16Pad + wd], v);
    } else {
      if (v & 0xFFFFu) atomicAdd(&g[p * kB16Pad + 2 * wd], v & 0xFFFFu);
      if (v >> 16) atomicAdd(&g[p * kB16Pad + 2 * wd + 1], v >> 16);
    }
  }

  // Fixed XOR butterfly within each wave, then the waves in order.
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    TailPart x = mine[p];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      TailPart o;
      o.sum_abs = __shfl_xor(x.sum_abs, m);
      o.sum_prob = __shfl_xor(x.sum_prob, m);
      o.max_key = (uint64_t)__shfl_xor((long long)x.max_key, m);
      o.max_pos = __shfl_xor(x.max_pos, m);
      o.count = __shfl_xor(x.count, m);
      x = tail_part_combine(x, o);
    }
    if (lane == 0) red[p][tid >> 6] = x;
    __builtin_amdgcn_sched_barrier(0);  // one pair at a time: fewer live registers
  }
  __syncthreads();
  if (tid < 3) {
    TailPart x = red[tid][0];
#pragma unroll
    for (int v = 1; v < kTailThreads / 64; ++v) x = tail_part_combine(x, red[tid][v]);
    w.part[n * 3 + tid] = x;
  }
}

// The rank target j of a pair wants among its `total` counted tokens (0:
// none): the two neighbours of each quantile, or the k-th largest (the
// smallest when fewer are counted).
__device__ __forceinline__ int64_t tail_target_rank(int j, int64_t total, int32_t k) {
  if (total <= 0) return 0;
  if (j < kWorstT) {
    int64_t lo, hi;
    quantile_ranks(total, quantile_prob(j >> 1), &lo, &hi);
    return (j & 1) ? hi : lo;
  }
  return k > 0 ? (total > k ? total - k + 1 : 1) : 0;
}

constexpr int kSelThreads = 1024;
constexpr int kS0Per = (kKeyBuckets + kSelThreads - 1) / kSelThreads;  // 5 buckets a thread

// Select after pass 0, one workgroup per pair: thread j sums the copies of
// buckets [5 j, 5 j + 5); a scan over the threads gives each target's bucket
// and its rank inside it. Thread 0 then plans pass 1 for the pair's targets:
// sources, list regions (each split by copy, at the offsets the copies'
// counts give) and gathers.
template <int kTP>
__global__ __launch_bounds__(kSelThreads) void tails_p0_select_kernel(TailWs w) {
  constexpr int kWaves = kSelThreads / 64;
  __shared__ int64_t s_wsum[kWaves], s_total;
  __shared__ int32_t s_bin[kTP];
  __shared__ int64_t s_rank[kTP], s_len[kTP], s_trank[kTP];
  __shared__ uint32_t s_sub[kTP][kCopies];
  __shared__ int32_t s_lreg[kTP];
  const int p = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kTP) s_bin[tid] = -1;
  uint32_t c[kS0Per];
  int64_t mine = 0;
#pragma unroll
  for (int j = 0; j < kS0Per; ++j) {
    const int b = tid * kS0Per + j;
    uint32_t s = 0u;
    if (b < kKeyBuckets) {
#pragma unroll
      for (int cp = 0; cp < kCopies; ++cp) s += w.hist0[(size_t)(cp * 3 + p) * kB16Pad + b];
    }
    c[j] = s;
    mine += s;
  }
  int64_t incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  if (tid == 0) {  // exclusive prefix of the wave sums, and the pair's total
    int64_t run = 0;
    for (int v = 0; v < kWaves; ++v) {
      const int64_t x = s_wsum[v];
      s_wsum[v] = run;
      run += x;
    }
    s_total = run;
    w.count[p] = run;
  }
  __syncthreads();
  incl += s_wsum[wave];
  if (tid < kTP) s_trank[tid] = tail_target_rank(tid, s_total, w.k);
  __syncthreads();
  const int64_t excl = incl - mine;
  for (int j = 0; j < kTP; ++j) {
    const int64_t rank = s_trank[j];
    if (rank > 0 && excl < rank && rank <= incl) {
      int64_t below = excl;
      int found = -1;
      uint32_t len = 0u;
#pragma unroll
      for (int q = 0; q < kS0Per; ++q) {
        if (found >= 0) continue;
        if (below + c[q] >= rank) {
          found = q;
          len = c[q];
        } else {
          below += c[q];
        }
      }
      const int b = tid * kS0Per + found;
      s_bin[j] = b;
      s_rank[j] = rank - below;
      s_len[j] = len;
#pragma unroll
      for (int cp = 0; cp < kCopies; ++cp) s_sub[j][cp] = w.hist0[(size_t)(cp * 3 + p) * kB16Pad + b];
    }
  }
  __syncthreads();
  if (tid != 0) return;
  // Bucket 0 holds only the key 0: a target there is selected. A source's
  // list region is cut from its pair's key buffer while it lasts.
  uint32_t hist = 0u, gath = 0u, own = 0u;
  int64_t used = 0;
  for (int j = 0; j < kTP; ++j) {
    const int u = kTP * p + j;
    const int b = s_bin[j];
    TailSel s{0ull, 0, -1, -1, 0, 0};
    int src = j;
    if (b > 0) {
      s.prefix = bucket_top16((uint32_t)b);
      s.rank = s_rank[j];
      for (int v = 0; v < j; ++v)
        if (s_bin[v] == b) {
          src = v;
          break;
        }
      if (src == j) {
        const int64_t len = s_len[j];
        if (len <= kGather) {
          gath |= 1u << u;
        } else {
          hist |= 1u << u;
          if (used + len <= w.cap) {
            own |= 1u << u;
            const int64_t off = p * w.cap + used;
            w.list[u] = TailList{off, len};
            int64_t o = off;
            for (int cp = 0; cp < kCopies; ++cp) {
              w.fill[(u * kCopies + cp) * kCtrStride64] = o;
              o += s_sub[j][cp];
            }
            used += len;
            s.lreg = u;
          }
        }
      } else {
        s.lreg = s_lreg[src];
      }
    }
    s_lreg[j] = s.lreg;
    w.sel[u] = s;
    w.plan->pre[u] = s.prefix;
    w.plan->src[u] = (int8_t)(kTP * p + src);
    w.plan->lsrc[u] = -1;  // pass 1 reads the batch
  }
  // The init kernel cleared the masks; each pair adds its sources.
  if (hist) atomicOr(&w.plan->hist, hist);
  if (gath) atomicOr(&w.plan->gath, gath);
  if (own) atomicOr(&w.plan->own, own);
}

// Appends the hitting lanes' keys to source t's gather buffer (one atomic
// for the wave). The select only plans a gather for at most kGather keys.
__device__ __forceinline__ void gather_add(const TailWs& w, int t, uint64_t key, bool hit, int lane) {
  const uint64_t hb = __ballot(hit);
  if (hb == 0) return;
  const int first = __ffsll((long long)hb) - 1;
  uint32_t base = 0u;
  if (lane == first) base = atomicAdd(&w.gcnt[t * kCtrStride32], (uint32_t)__popcll(hb));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, first);
  const uint32_t e = base + lanes_below(hb);
  if (hit && e < (uint32_t)kGather) w.gbuf[(size_t)t * kGather + e] = key;
}

// Pass 1 over one row per workgroup: each histogram source counts byte
// [47:40] of the keys in its bucket, each source with a list region copies
// them into it, each gathering source gathers them. Copies go in chunks of
// 1 024 positions: every wave numbers its hits per source from its ballots
// (no atomics), the waves' counts are laid end to end, one atomic per source
// reserves the chunk's span of the region part that this workgroup's copy
// counted, and the keys, still in registers, are written. The byte
// histograms are 16-bit counters, two to a word, for rows of at most 65 535
// positions (kWide false; a bin counts at most L keys), else 32-bit.
template <bool kVec, bool kWide, int kTP>
__global__ __launch_bounds__(kTailThreads) void tails_p1_kernel(TailArgs a, TailWs w) {
  constexpr int kNT = 3 * kTP;
  constexpr int kW = kTailThreads / 64;
  constexpr int kRow = kWide ? 256 : 128;  // words per source histogram
  __shared__ uint32_t h[kNT * kRow];
  __shared__ uint32_t s_wcnt[kW][kNT];
  __shared__ int64_t s_wbase[kW][kNT], s_lim[kNT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t hist = w.plan->hist, gath = w.plan->gath, own = w.plan->own;
  const uint32_t act = hist | gath;
  if (act == 0u) return;  // uniform
  uint64_t pre[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) pre[t] = w.plan->pre[t];
#pragma unroll
  for (int t = 0; t < kNT; ++t)
    if (((hist >> t) & 1u) && tid < kRow) h[t * kRow + tid] = 0u;
  if (tid < kNT) {
    const TailList R = w.list[tid];
    s_lim[tid] = R.off + R.len;
  }
  __syncthreads();

  const int64_t n = blockIdx.x;
  const int cp = (int)(n % kCopies);
  const float* const rows[3] = {a.A + n * a.ld, a.B + n * a.ld, a.C + n * a.ld};
  const uint8_t* M = a.mask + n * a.ld;
  constexpr int64_t kStep = 4 * kTailThreads;
  const int64_t Lw = (a.L + kStep - 1) / kStep * kStep;
  for (int64_t i0 = 4 * (int64_t)tid; i0 < Lw; i0 += kStep) {
    float vv[4][3];
    bool actv[4];
    tail_load4<kVec>(a, rows, M, i0, vv, actv);
    uint64_t key[4][3];
    uint32_t okm[3] = {0u, 0u, 0u};
    uint32_t slot[4][3];  // index among the wave's hits of the source
    int tsel[4][3];       // the source that copies the key (-1: none)
    uint32_t wrun[kNT];   // the wave's hits per source so far (uniform)
#pragma unroll
    for (int t = 0; t < kNT; ++t) wrun[t] = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        okm[p] |= tail_key(vv[k], actv[k], p, &key[k][p]) ? 1u << k : 0u;
        tsel[k][p] = -1;
        slot[k][p] = 0u;
      }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
#pragma unroll
      for (int j = 0; j < kTP; ++j) {
        const int t = kTP * p + j;
        if (!((act >> t) & 1u)) continue;  // uniform
        uint32_t hm = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          hm |= (((okm[p] >> k) & 1u) && (key[k][p] >> 48) == pre[t]) ? 1u << k : 0u;
        if (__ballot(hm != 0u) == 0) continue;  // uniform: no key of the wave in the bucket
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bool hit = (hm >> k) & 1u;
          if ((hist >> t) & 1u)
            hist16_add<kWide>(h + t * kRow, (uint32_t)(key[k][p] >> 40) & 255u, hit, lane);
          if ((gath >> t) & 1u) gather_add(w, t, key[k][p], hit, lane);
          if ((own >> t) & 1u) {
            const uint64_t hb = __ballot(hit);
            if (hit) {
              slot[k][p] = wrun[t] + lanes_below(hb);
              tsel[k][p] = t;
            }
            wrun[t] += (uint32_t)__popcll(hb);
          }
        }
      }
    }
    if (own != 0u) {  // uniform
      if (lane == 0) {
#pragma unroll
        for (int t = 0; t < kNT; ++t)
          if ((own >> t) & 1u) s_wcnt[wave][t] = wrun[t];
      }
      __syncthreads();
      if (tid < kNT && ((own >> tid) & 1u)) {
        uint32_t tot = 0u;
#pragma unroll
        for (int v = 0; v < kW; ++v) tot += s_wcnt[v][tid];
        int64_t b = (int64_t)atomicAdd(reinterpret_cast<unsigned long long*>(&w.fill[(tid * kCopies + cp) * kCtrStride64]),
                                       (unsigned long long)tot);
#pragma unroll
        for (int v = 0; v < kW; ++v) {
          s_wbase[v][tid] = b;
          b += s_wcnt[v][tid];
        }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          const int t = tsel[k][p];
          if (t < 0) continue;
          const int64_t e = s_wbase[wave][t] + slot[k][p];
          if (e < s_lim[t]) w.keys[e] = key[k][p];
        }
    }
  }
  __syncthreads();
  uint32_t* hc = w.hist + (size_t)cp * kHistStride;
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    if (!((hist >> t) & 1u)) continue;  // uniform
    if (kWide) {
      const uint32_t v = h[t * kRow + tid];
      if (v) atomicAdd(&hc[t * 256 + tid], v);
    } else {
      // Bin tid is half (tid & 1) of word tid >> 1.
      const uint32_t v = (h[t * kRow + (tid >> 1)] >> ((tid & 1) << 4)) & 0xFFFFu;
      if (v) atomicAdd(&hc[t * 256 + tid], v);
    }
  }
}

// Select after pass p >= 1, by one workgroup of kThreads (every thread
// calls it; cnt is kNT x 256 words of LDS). Phase 1 sums the copies of every
// histogram source into LDS, phase 2 clears them, phase 3 finds the bin that
// holds each live target's rank (one wave per target in turn, 4 bins a
// lane); the targets of a source that gathered in this pass are handed to
// the finish. Thread 0 then plans the next pass: a source with at most
// kGather keys under its prefix gathers them, the others histogram.
template <int kTP, int kThreads>
__device__ void tails_select_byte(const TailWs& w, int pass, uint32_t (*cnt)[256]) {
  constexpr int kNT = 3 * kTP;
  constexpr int kWaves = kThreads / 64;
  __shared__ uint64_t s_pre[kNT];
  __shared__ int64_t s_rank[kNT], s_len[kNT];
  __shared__ int s_src[kNT], s_lreg[kNT], s_fin[kNT];
  __shared__ uint32_t s_hm, s_gm;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int shift = pass_shift(pass);
  if (threadIdx.x < kNT) {
    const int u = threadIdx.x;
    const TailSel x = w.sel[u];
    s_pre[u] = w.plan->pre[u];
    s_src[u] = w.plan->src[u];
    s_rank[u] = x.rank;
    s_lreg[u] = x.lreg;
    s_fin[u] = x.fin_src;
    s_len[u] = 0;
  }
  if (threadIdx.x == 0) {
    s_hm = w.plan->hist;
    s_gm = w.plan->gath;
  }
  __syncthreads();
  const uint32_t hm = s_hm, gm = s_gm;
  if ((hm | gm) == 0u) return;  // uniform: the pass had nothing to do
  for (int t = wave; t < kNT; t += kWaves) {
    if (!((hm >> t) & 1u)) continue;
    uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int cp = 0; cp < kCopies; ++cp) {
      const uint4 q = *reinterpret_cast<const uint4*>(w.hist + cp * kHistStride + t * 256 + 4 * lane);
      c[0] += q.x;
      c[1] += q.y;
      c[2] += q.z;
      c[3] += q.w;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) cnt[t][4 * lane + k] = c[k];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kCopies * kNT * 64; i += kThreads) {
    const int cp = i / (kNT * 64), r = i % (kNT * 64);
    if ((hm >> (r >> 6)) & 1u)
      *reinterpret_cast<uint4*>(w.hist + cp * kHistStride + 4 * r) = make_uint4(0u, 0u, 0u, 0u);
  }
  for (int t = wave; t < kNT; t += kWaves) {
    const int64_t rank = s_rank[t];
    if (rank <= 0 || s_fin[t] >= 0) continue;  // uniform: done, none, or finishing
    const int src = s_src[t];
    if ((gm >> src) & 1u) {
      if (lane == 0) {
        s_fin[t] = src;
        w.sel[t].fin_src = src;
        w.sel[t].fin_bits = shift + 8;
      }
      continue;
    }
    if (!((hm >> src) & 1u)) continue;
    uint32_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = cnt[src][4 * lane + k];
    const int64_t lsum = (int64_t)c[0] + c[1] + c[2] + c[3];
    int64_t incl = lsum;  // inclusive scan over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int64_t excl = incl - lsum;
    if (excl < rank && rank <= incl) {
      int64_t below = excl;
      int k = 0;
      while (below + (int64_t)c[k] < rank) below += c[k++];
      const uint64_t np = (s_pre[t] << 8) | (uint64_t)(4 * lane + k);
      w.sel[t].prefix = np;
      w.sel[t].rank = rank - below;
      s_pre[t] = np;
      s_rank[t] = rank - below;
      s_len[t] = (int64_t)c[k];
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  uint32_t hist = 0u, gath = 0u;
  for (int u = 0; u < kNT; ++u) {
    const bool live = s_rank[u] > 0 && s_fin[u] < 0;
    int src = u;
    if (live) {
      for (int v = kTP * (u / kTP); v < u; ++v)
        if (s_rank[v] > 0 && s_fin[v] < 0 && s_pre[v] == s_pre[u]) {
          src = v;
          break;
        }
      if (src == u && pass < kLastPass) {
        if (s_len[u] <= kGather) gath |= 1u << u;
        else hist |= 1u << u;
      }
    }
    w.plan->pre[u] = s_pre[u];
    w.plan->src[u] = (int8_t)src;
    w.plan->lsrc[u] = s_lreg[u];
  }
  w.plan->hist = hist;
  w.plan->gath = gath;
  w.plan->own = 0u;
}

template <int kTP>
__global__ __launch_bounds__(kSelThreads) void tails_select_kernel(TailWs w, int pass) {
  __shared__ uint32_t cnt[3 * kTP][256];
  tails_select_byte<kTP, kSelThreads>(w, pass, cnt);
}

// Passes 2 .. 6: each histogram source counts this pass's byte of the keys
// under its prefix, each gathering source gathers them, reading its list
// region (grid-stride over whole waves: the ballots need every lane), or the
// batch (sequences dealt to the workgroups in turn) for a source without
// one. Integer counts, so the order of the keys does not matter.
constexpr int kListBlocks = 512;

template <bool kVec, int kTP>
__global__ __launch_bounds__(kTailThreads) void tails_list_kernel(TailArgs a, TailWs w, int pass) {
  constexpr int kNT = 3 * kTP;
  __shared__ uint32_t h[kNT * 256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int shift = pass_shift(pass);
  const uint32_t hist = w.plan->hist, gath = w.plan->gath;
  const uint32_t act = hist | gath;
  if (act == 0u) return;  // uniform: no target left for the passes
  uint64_t pre[kNT];
  int lst[kNT];
  uint32_t batch = 0u;
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    pre[t] = w.plan->pre[t];
    lst[t] = w.plan->lsrc[t];
    if (((act >> t) & 1u) && lst[t] < 0) batch |= 1u << t;
  }
#pragma unroll
  for (int t = 0; t < kNT; ++t)
    if ((hist >> t) & 1u) h[t * 256 + tid] = 0u;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * kTailThreads;
  const int64_t wave0 = (int64_t)blockIdx.x * kTailThreads + (tid - lane);
  for (int u = 0; u < kNT; ++u) {
    bool used = false;
#pragma unroll
    for (int t = 0; t < kNT; ++t) used = used || (((act >> t) & 1u) && lst[t] == u);
    if (!used) continue;  // uniform
    const TailList R = w.list[u];
    for (int64_t e0 = wave0; e0 < R.len; e0 += stride) {
      const int64_t e = e0 + lane;
      const bool in = e < R.len;
      const uint64_t key = in ? w.keys[R.off + e] : 0ull;
      const uint32_t digit = (uint32_t)(key >> shift) & 255u;
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        if (!((act >> t) & 1u) || lst[t] != u) continue;  // uniform
        const bool hit = in && (key >> (shift + 8)) == pre[t];
        if ((hist >> t) & 1u) wave_hist_add(h + t * 256, digit, hit, lane);
        else gather_add(w, t, key, hit, lane);
      }
    }
  }
  if (batch != 0u) {  // uniform
    constexpr int64_t kStep = 4 * kTailThreads;
    const int64_t Lw = (a.L + kStep - 1) / kStep * kStep;
    for (int64_t n = blockIdx.x; n < a.N; n += gridDim.x) {
      const float* const rows[3] = {a.A + n * a.ld, a.B + n * a.ld, a.C + n * a.ld};
      const uint8_t* M = a.mask + n * a.ld;
      for (int64_t i0 = 4 * (int64_t)tid; i0 < Lw; i0 += kStep) {
        float vv[4][3];
        bool actv[4];
        tail_load4<kVec>(a, rows, M, i0, vv, actv);
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int p = 0; p < 3; ++p) {
            uint64_t key;
            const bool ok = tail_key(vv[k], actv[k], p, &key);
            const uint32_t digit = (uint32_t)(key >> shift) & 255u;
#pragma unroll
            for (int j = 0; j < kTP; ++j) {
              const int t = kTP * p + j;
              if (!((batch >> t) & 1u)) continue;  // uniform
              const bool hit = ok && (key >> (shift + 8)) == pre[t];
              if ((hist >> t) & 1u) wave_hist_add(h + t * 256, digit, hit, lane);
              else gather_add(w, t, key, hit, lane);
            }
          }
      }
    }
  }
  __syncthreads();
  uint32_t* hc = w.hist + (size_t)(blockIdx.x % kCopies) * kHistStride;
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    if (!((hist >> t) & 1u)) continue;  // uniform
    const uint32_t v = h[t * 256 + tid];
    if (v) atomicAdd(&hc[t * 256 + tid], v);
  }
}

constexpr int kFinThreads = 1024;
static_assert(kFinThreads * 4 == kGather, "four gathered keys a thread");

// The finish of source s (every thread of a kFinThreads workgroup calls it):
// its targets' remaining bytes are selected from its gathered keys, held
// four to a thread, one byte per round (histograms in LDS, one wave per
// target). Does nothing unless a target of s was handed to it.
template <int kTP>
__device__ void tails_finish_source(const TailWs& w, int s) {
  __shared__ uint32_t hh[kTP][256];
  __shared__ uint64_t s_pre[kTP];
  __shared__ int64_t s_rank[kTP];
  __shared__ uint32_t s_mine;
  __shared__ int s_bits;
  const int p = s / kTP, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __syncthreads();  // the previous source's readers are done with the LDS
  if (tid == 0) {
    uint32_t m = 0u;
    int bits = 0;
    for (int j = 0; j < kTP; ++j) {
      const TailSel x = w.sel[kTP * p + j];
      s_pre[j] = x.prefix;
      s_rank[j] = x.rank;
      if (x.fin_src == s && x.rank > 0) {
        m |= 1u << j;
        bits = x.fin_bits;
      }
    }
    s_mine = m;
    s_bits = bits;
  }
  __syncthreads();
  const uint32_t mine = s_mine;
  if (mine == 0u) return;  // uniform
  const uint32_t g = min(w.gcnt[s * kCtrStride32], (uint32_t)kGather);
  uint64_t key[4];
  bool in[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t i = (uint32_t)(tid + m * kFinThreads);
    in[m] = i < g;
    key[m] = in[m] ? w.gbuf[(size_t)s * kGather + i] : 0ull;
  }
  for (int sh = s_bits - 8; sh >= 0; sh -= 8) {
    for (int i = tid; i < kTP * 256; i += kFinThreads) hh[i >> 8][i & 255] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTP; ++j) {
      if (!((mine >> j) & 1u)) continue;  // uniform
      const uint64_t pj = s_pre[j];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        wave_hist_add(hh[j], (uint32_t)(key[m] >> sh) & 255u, in[m] && (key[m] >> (sh + 8)) == pj,
                      lane);
    }
    __syncthreads();
    for (int j = wave; j < kTP; j += kFinThreads / 64) {
      if (!((mine >> j) & 1u)) continue;
      const int64_t rank = s_rank[j];
      uint32_t c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = hh[j][4 * lane + k];
      const int64_t lsum = (int64_t)c[0] + c[1] + c[2] + c[3];
      int64_t incl = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const int64_t excl = incl - lsum;
      if (excl < rank && rank <= incl) {
        int64_t below = excl;
        int k = 0;
        while (below + (int64_t)c[k] < rank) below += c[k++];
        s_pre[j] = (s_pre[j] << 8) | (uint64_t)(4 * lane + k);
        s_rank[j] = rank - below;
      }
    }
    __syncthreads();
  }
  if (tid < kTP && ((mine >> tid) & 1u)) {
    w.sel[kTP * p + tid].prefix = s_pre[tid];
    w.sel[kTP * p + tid].rank = 0;
  }
}

// One workgroup per source (most exit at once).
template <int kTP>
__global__ __launch_bounds__(kFinThreads) void tails_finish_kernel(TailWs w) {
  tails_finish_source<kTP>(w, blockIdx.x);
}

// Batch results. Workgroup p < 3 reduces pair p's per-sequence partials
// (after the finish): thread j folds the
// contiguous sequences [j per, (j + 1) per) in order (per depends on N
// only), then a fixed XOR butterfly within each wave and the waves in order.
// The maximum keeps the first sequence (and, within it, the first column)
// that reaches it. Workgroups 3, 4, ... fold the position profile's chunks:
// four fixed groups of consecutive chunks, each in order, then the groups in
// order.
template <int kTP>
__global__ __launch_bounds__(kFinThreads) void tails_final_kernel(TailArgs a, TailWs w) {
  if (blockIdx.x >= 3) {
    // Thread (q, o) of a workgroup folds the chunks [q G, (q + 1) G) of output
    // o of its 256 (G = ceil(nch / 4)); thread (0, o) then adds the four
    // partials in order.
    __shared__ double fs[4][kFinThreads / 4];
    __shared__ int32_t fk[4][kFinThreads / 4];
    const int q = threadIdx.x / (kFinThreads / 4), o = threadIdx.x % (kFinThreads / 4);
    const int G = (w.nch + 3) / 4;
    const int c0 = q * G, c1 = min(w.nch, c0 + G);
    for (int64_t base = (int64_t)(blockIdx.x - 3) * (kFinThreads / 4); base < 3 * a.L;
         base += (int64_t)(gridDim.x - 3) * (kFinThreads / 4)) {  // uniform
      const int64_t idx = base + o;  // p * L + i
      double s = 0.0;
      int32_t k = 0;
      if (idx < 3 * a.L) {
#pragma unroll 8
        for (int c = c0; c < c1; ++c) {
          s += w.pos_part[(size_t)c * 3 * a.L + idx];
          k += w.pos_cpart[(size_t)c * 3 * a.L + idx];
        }
      }
      fs[q][o] = s;
      fk[q][o] = k;
      __syncthreads();
      if (q == 0 && idx < 3 * a.L) {
        a.pos_sum[idx] = ((fs[0][o] + fs[1][o]) + fs[2][o]) + fs[3][o];
        a.pos_count[idx] = fk[0][o] + fk[1][o] + fk[2][o] + fk[3][o];
      }
      __syncthreads();
    }
    return;
  }
  constexpr int kWaves = kFinThreads / 64;
  __shared__ TailPart red[kWaves];
  __shared__ int32_t red_seq[kWaves];
  const int p = blockIdx.x, tid = threadIdx.x, lane = tid & 63;

  const int64_t per = (a.N + kFinThreads - 1) / kFinThreads;
  TailPart x{0.0, 0.0, 0ull, -1, 0};
  int32_t xs = -1;
  const int64_t lo = tid * per, hi = min(a.N, lo + per);
#pragma unroll 4
  for (int64_t n = lo; n < hi; ++n) {
    const TailPart y = w.part[n * 3 + p];
    x.sum_abs += y.sum_abs;
    x.sum_prob += y.sum_prob;
    x.count += y.count;
    if (y.max_pos >= 0 && (x.max_pos < 0 || y.max_key > x.max_key)) {  // n ascends
      x.max_key = y.max_key;
      x.max_pos = y.max_pos;
      xs = (int32_t)n;
    }
  }
  // Both lanes of a butterfly step get the same result: sums are added in
  // either order to the same value, and equal maxima keep the lower sequence.
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    TailPart o;
    o.sum_abs = __shfl_xor(x.sum_abs, m);
    o.sum_prob = __shfl_xor(x.sum_prob, m);
    o.count = __shfl_xor(x.count, m);
    o.max_key = (uint64_t)__shfl_xor((long long)x.max_key, m);
    o.max_pos = __shfl_xor(x.max_pos, m);
    const int32_t os = __shfl_xor(xs, m);
    x.sum_abs += o.sum_abs;
    x.sum_prob += o.sum_prob;
    x.count += o.count;
    if (o.max_pos >= 0 &&
        (x.max_pos < 0 || o.max_key > x.max_key || (o.max_key == x.max_key && os < xs))) {
      x.max_key = o.max_key;
      x.max_pos = o.max_pos;
      xs = os;
    }
  }
  if (lane == 0) {
    red[tid >> 6] = x;
    red_seq[tid >> 6] = xs;
  }
  __syncthreads();
  if (tid != 0) return;
  TailPart r = red[0];
  int32_t rs = red_seq[0];
  for (int v = 1; v < kWaves; ++v) {  // waves in order: lower sequences first
    const TailPart& y = red[v];
    r.sum_abs += y.sum_abs;
    r.sum_prob += y.sum_prob;
    r.count += y.count;
    if (y.max_pos >= 0 &&
        (r.max_pos < 0 || y.max_key > r.max_key || (y.max_key == r.max_key && red_seq[v] < rs))) {
      r.max_key = y.max_key;
      r.max_pos = y.max_pos;
      rs = red_seq[v];
    }
  }
  lp_tail_stats o;
  o.count = w.count[p];
  const bool any = o.count > 0;
  double q[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const double qlo = __longlong_as_double((long long)w.sel[kTP * p + 2 * j].prefix);
    const double qhi = __longlong_as_double((long long)w.sel[kTP * p + 2 * j + 1].prefix);
    q[j] = any ? quantile_lerp(o.count, quantile_prob(j), qlo, qhi) : 0.0;
  }
  o.q50 = q[0];
  o.q95 = q[1];
  o.q99 = q[2];
  o.max_abs = any ? __longlong_as_double((long long)r.max_key) : 0.0;
  o.max_seq = any ? rs : -1;
  o.max_pos = any ? r.max_pos : -1;
  o.sum_abs = r.sum_abs;
  o.sum_prob_abs = r.sum_prob;
  a.out[p] = o;
}

// ---- Worst k tokens ----------------------------------------------------

// Threshold of pair p: the key its k-th-largest target selected (meaningful
// when the pair counts any token).
__device__ __forceinline__ uint64_t worst_tau(const TailWs& w, int p) {
  return w.sel[kMaxTP * p + kWorstT].prefix;  // only with kTP == kMaxTP
}

// Per sequence and pair: counted tokens with key > tau and key == tau.
template <bool kVec>
__global__ __launch_bounds__(kTailThreads) void tails_worst_count_kernel(TailArgs a, TailWs w) {
  __shared__ uint32_t tot[6];
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 6) tot[tid] = 0u;
  __syncthreads();
  uint64_t tau[3];
  bool on[3];
  uint32_t known[3];  // the equal count when the row need not be read
  const int64_t n = blockIdx.x;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    tau[p] = worst_tau(w, p);
    // Pass 0 kept the sequence's largest key and its token count: with the
    // largest key below tau no token counts; with tau and the largest key
    // both 0, every counted token equals tau and none is above it.
    const TailPart q = w.part[n * 3 + p];
    const bool any = w.count[p] > 0 && q.max_pos >= 0 && q.max_key >= tau[p];
    const bool zeros = any && tau[p] == 0ull && q.max_key == 0ull;
    on[p] = any && !zeros;
    known[p] = zeros ? (uint32_t)q.count : 0u;
  }
  if (!(on[0] || on[1] || on[2])) {  // uniform: nothing to read
    if (tid < 3) {
      w.wcnt[tid * a.N + n] = 0u;
      w.wcnt[(3 + tid) * a.N + n] = known[tid];
    }
    return;
  }
  const float* const rows[3] = {a.A + n * a.ld, a.B + n * a.ld, a.C + n * a.ld};
  const uint8_t* M = a.mask + n * a.ld;
  uint32_t c[6] = {0u, 0u, 0u, 0u, 0u, 0u};
  constexpr int64_t kStep = 4 * kTailThreads;
  for (int64_t i0 = 4 * (int64_t)tid; i0 < a.L; i0 += kStep) {
    float vv[4][3];
    bool actv[4];
    tail_load4<kVec>(a, rows, M, i0, vv, actv);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const float l = vv[k][pair_left(p)], r = vv[k][pair_right(p)];
        if (!(on[p] && actv[k] && __builtin_isfinite(l) && __builtin_isfinite(r))) continue;
        const uint64_t key = (uint64_t)__double_as_longlong(fabs((double)l - (double)r));
        c[p] += key > tau[p] ? 1u : 0u;
        c[3 + p] += key == tau[p] ? 1u : 0u;
      }
  }
  // Integer sums: the order of the additions does not matter.
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    uint32_t v = c[q];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off);
    if (lane == 0 && v) atomicAdd(&tot[q], v);
  }
  __syncthreads();
  if (tid < 6) {
    const uint32_t kn = tid < 3 ? 0u : (tid == 3 ? known[0] : (tid == 4 ? known[1] : known[2]));
    w.wcnt[tid * a.N + n] = tot[tid] + kn;  // a pair not read has tot 0
  }
}

// Exclusive scans of the six count rows over the sequences, one workgroup
// per row, 64-bit offsets. Thread j takes the contiguous sequences
// [j per, (j + 1) per).
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void tails_worst_scan_kernel(TailWs w, int64_t N) {
  __shared__ int64_t wsum[kScanThreads / 64];
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* cnt = w.wcnt + q * N;
  int64_t* off = w.woff + q * N;
  const int64_t per = (N + kScanThreads - 1) / kScanThreads;
  const int64_t lo = min(N, tid * per), hi = min(N, lo + per);
  int64_t tot = 0;
  for (int64_t n = lo; n < hi; ++n) tot += cnt[n];
  int64_t incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int64_t run = incl - tot;
  for (int v = 0; v < wave; ++v) run += wsum[v];
  for (int64_t n = lo; n < hi; ++n) {
    off[n] = run;
    run += cnt[n];
  }
}

// Inclusive scan of one value over the workgroup's threads, in thread order;
// `total` is the workgroup's sum. Every thread must call it.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = (uint32_t)__shfl_up((int)incl, o);
    if (lane >= o) incl += u;
  }
  __syncthreads();  // the previous call's readers are done with wsum
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0u;
  total = 0u;
#pragma unroll
  for (int x = 0; x < kTailThreads / 64; ++x) {
    before += x < wave ? wsum[x] : 0u;
    total += wsum[x];
  }
  return before + incl;
}

// Writes the candidates: every token above tau at its slot, and the tokens
// equal to tau whose row-major rank among them is below what k still needs.
// Slots follow position order within the sequence (threads take four
// consecutive positions, in thread order, per 1024-position chunk).
template <bool kVec>
__global__ __launch_bounds__(kTailThreads) void tails_worst_write_kernel(TailArgs a, TailWs w) {
  __shared__ uint32_t wsum[kTailThreads / 64];
  const int tid = threadIdx.x;
  const int64_t n = blockIdx.x, N = a.N;
  uint64_t tau[3];
  bool on[3];
  int64_t gt_total[3], need_eq[3], run_g[3], run_e[3], m[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    tau[p] = worst_tau(w, p);
    on[p] = w.count[p] > 0;
    m[p] = min((int64_t)w.k, w.count[p]);
    gt_total[p] = w.woff[p * N + N - 1] + w.wcnt[p * N + N - 1];
    need_eq[p] = m[p] - gt_total[p];
    run_g[p] = w.woff[p * N + n];
    run_e[p] = w.woff[(3 + p) * N + n];
  }
  // A sequence with no token above tau, and none equal to it that k still
  // needs (its first one would rank at or past need_eq), writes nothing and
  // skips its row (every thread reads the same counts: uniform).
  bool any = false;
#pragma unroll
  for (int p = 0; p < 3; ++p)
    any = any || (on[p] && (w.wcnt[p * N + n] > 0u ||
                            (w.wcnt[(3 + p) * N + n] > 0u && run_e[p] < need_eq[p])));
  if (!any) return;
  const float* const rows[3] = {a.A + n * a.ld, a.B + n * a.ld, a.C + n * a.ld};
  const uint8_t* M = a.mask + n * a.ld;
  constexpr int64_t kStep = 4 * kTailThreads;
  const int64_t Lw = (a.L + kStep - 1) / kStep * kStep;  // every thread takes every chunk
  for (int64_t i0 = 4 * (int64_t)tid; i0 < Lw; i0 += kStep) {
    float vv[4][3];
    bool actv[4];
    tail_load4<kVec>(a, rows, M, i0, vv, actv);
    uint64_t key[4][3];
    uint32_t fg[3] = {0u, 0u, 0u}, fe[3] = {0u, 0u, 0u};  // bit k: position i0 + k is above / equal
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const float l = vv[k][pair_left(p)], r = vv[k][pair_right(p)];
        const bool ok = on[p] && actv[k] && __builtin_isfinite(l) && __builtin_isfinite(r);
        key[k][p] = (uint64_t)__double_as_longlong(fabs((double)l - (double)r));
        fg[p] |= (ok && key[k][p] > tau[p]) ? 1u << k : 0u;
        fe[p] |= (ok && key[k][p] == tau[p]) ? 1u << k : 0u;
      }
    // Few tokens reach tau: a chunk without any skips its scans (the test is
    // uniform over the workgroup, so every thread takes the same branch).
    if (!__syncthreads_or((fg[0] | fg[1] | fg[2] | fe[0] | fe[1] | fe[2]) != 0u)) continue;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      uint32_t tg, te;
      const uint32_t ig = block_incl_scan((uint32_t)__popc(fg[p]), wsum, tg);
      const uint32_t ie = block_incl_scan((uint32_t)__popc(fe[p]), wsum, te);
      int64_t sg = run_g[p] + ig - (uint32_t)__popc(fg[p]);
      int64_t se = run_e[p] + ie - (uint32_t)__popc(fe[p]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int32_t pos = (int32_t)(i0 + k);
        if (fg[p] & (1u << k)) {
          if (sg < m[p]) w.cand[(int64_t)p * w.k + sg] = WorstCand{key[k][p], (int32_t)n, pos};
          ++sg;
        }
        if (fe[p] & (1u << k)) {
          if (se < need_eq[p])
            w.cand[(int64_t)p * w.k + gt_total[p] + se] = WorstCand{key[k][p], (int32_t)n, pos};
          ++se;
        }
      }
      run_g[p] += tg;
      run_e[p] += te;
    }
  }
}

// One workgroup per pair: bitonic sort of the candidates (|delta| descending,
// then sequence, then column ascending) and the output rows; rows past the
// counted tokens get |delta| 0 and sequence and column -1.
constexpr int kWorstSortThreads = 1024;

__device__ __forceinline__ bool worst_before(const WorstCand& x, const WorstCand& y) {
  if (x.key != y.key) return x.key > y.key;
  if (x.seq != y.seq) return x.seq < y.seq;
  return x.pos < y.pos;
}

__global__ __launch_bounds__(kWorstSortThreads) void tails_worst_sort_kernel(TailArgs a, TailWs w) {
  __shared__ WorstCand s[LP_WORST_MAX];
  const int p = blockIdx.x, tid = threadIdx.x;
  const int64_t m = min((int64_t)w.k, w.count[p]);
  int P = 1;
  while (P < m) P <<= 1;
  // Padding sorts last: |delta| 0 and the largest sequence index.
  for (int i = tid; i < P; i += kWorstSortThreads)
    s[i] = i < m ? w.cand[(int64_t)p * w.k + i] : WorstCand{0ull, 0x7FFFFFFF, 0x7FFFFFFF};
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += kWorstSortThreads) {
        const int j = i ^ stride;
        if (j > i) {
          // Blocks with (i & size) == 0 end in the wanted order, the others
          // in the reverse; the last merge (size == P) orders everything.
          const bool fwd = (i & size) == 0;
          const WorstCand x = s[i], y = s[j];
          if (worst_before(y, x) == fwd) {
            s[i] = y;
            s[j] = x;
          }
        }
      }
      __syncthreads();
    }
  for (int i = tid; i < w.k; i += kWorstSortThreads) {
    lp_worst_token o;
    if (i < m) {
      o.abs_delta = __longlong_as_double((long long)s[i].key);
      o.seq = s[i].seq;
      o.pos = s[i].pos;
    } else {
      o.abs_delta = 0.0;
      o.seq = -1;
      o.pos = -1;
    }
    a.worst[(int64_t)p * w.k + i] = o;
  }
}

}  // namespace

size_t tails_workspace_bytes(int64_t N, int64_t L, int32_t k) { return tail_bytes(N, L, k); }

// The selection passes and the batch results, for kTP targets per pair.
template <int kTP>
static void launch_select(const TailArgs& a, const TailWs& w, hipStream_t stream) {
  const dim3 rows((unsigned)a.N), blk(kTailThreads);
  if (a.N > 0) {
    // Also with L == 0: pass 0 writes the empty partials.
    const bool wide = a.L > 65535;
    if (a.vec) {
      if (wide) hipLaunchKernelGGL((tails_p0_kernel<true, true>), rows, blk, 0, stream, a, w);
      else hipLaunchKernelGGL((tails_p0_kernel<true, false>), rows, blk, 0, stream, a, w);
    } else {
      if (wide) hipLaunchKernelGGL((tails_p0_kernel<false, true>), rows, blk, 0, stream, a, w);
      else hipLaunchKernelGGL((tails_p0_kernel<false, false>), rows, blk, 0, stream, a, w);
    }
  }
  // With no token the histograms are empty: count 0 and no rank to select.
  hipLaunchKernelGGL(tails_p0_select_kernel<kTP>, dim3(3), dim3(kSelThreads), 0, stream, w);
  if (a.N > 0 && a.L > 0) {
    const bool wide = a.L > 65535;
    if (a.vec) {
      if (wide) hipLaunchKernelGGL((tails_p1_kernel<true, true, kTP>), rows, blk, 0, stream, a, w);
      else hipLaunchKernelGGL((tails_p1_kernel<true, false, kTP>), rows, blk, 0, stream, a, w);
    } else {
      if (wide) hipLaunchKernelGGL((tails_p1_kernel<false, true, kTP>), rows, blk, 0, stream, a, w);
      else hipLaunchKernelGGL((tails_p1_kernel<false, false, kTP>), rows, blk, 0, stream, a, w);
    }
    hipLaunchKernelGGL(tails_select_kernel<kTP>, dim3(1), dim3(kSelThreads), 0, stream, w, 1);
    for (int pass = 2; pass <= kLastPass; ++pass) {
      if (a.vec)
        hipLaunchKernelGGL((tails_list_kernel<true, kTP>), dim3(kListBlocks), blk, 0, stream, a, w, pass);
      else
        hipLaunchKernelGGL((tails_list_kernel<false, kTP>), dim3(kListBlocks), blk, 0, stream, a, w, pass);
      hipLaunchKernelGGL(tails_select_kernel<kTP>, dim3(1), dim3(kSelThreads), 0, stream, w, pass);
    }
    hipLaunchKernelGGL(tails_finish_kernel<kTP>, dim3(3 * kTP), dim3(kFinThreads), 0, stream, w);
  }
  // Also the position profile's fold.
  const int64_t fold_all = a.pos_sum && a.L > 0 ? (3 * a.L + kFinThreads / 4 - 1) / (kFinThreads / 4) : 0;
  const unsigned fold = (unsigned)(fold_all < 65536 ? fold_all : 65536);  // then a grid-stride loop
  hipLaunchKernelGGL(tails_final_kernel<kTP>, dim3(3 + fold), dim3(kFinThreads), 0, stream, a, w);
}

hipError_t launch_tails(const TailArgs& a, hipStream_t stream) {
  const TailWs w = tail_layout(a.workspace, a.N, a.L, a.worst_k);
  // With the position profile asked for, its stage 1 (also with N == 0:
  // zero partials for the fold) runs in the init kernel.
  const bool pos = a.pos_sum && a.L > 0;
  const dim3 init_grid =
      pos ? dim3((unsigned)((a.L + kTailThreads - 1) / kTailThreads), (unsigned)w.nch) : dim3(kInitBlocks);
  hipLaunchKernelGGL(tails_init_kernel, init_grid, dim3(kTailThreads), 0, stream, a, w, pos);
  if (a.worst_k > 0) {
    launch_select<kMaxTP>(a, w, stream);
    if (a.N > 0 && a.L > 0) {
      if (a.vec) {
        hipLaunchKernelGGL(tails_worst_count_kernel<true>, dim3((unsigned)a.N), dim3(kTailThreads),
                           0, stream, a, w);
        hipLaunchKernelGGL(tails_worst_scan_kernel, dim3(6), dim3(kScanThreads), 0, stream, w, a.N);
        hipLaunchKernelGGL(tails_worst_write_kernel<true>, dim3((unsigned)a.N), dim3(kTailThreads),
                           0, stream, a, w);
      } else {
        hipLaunchKernelGGL(tails_worst_count_kernel<false>, dim3((unsigned)a.N), dim3(kTailThreads),
                           0, stream, a, w);
        hipLaunchKernelGGL(tails_worst_scan_kernel, dim3(6), dim3(kScanThreads), 0, stream, w, a.N);
        hipLaunchKernelGGL(tails_worst_write_kernel<false>, dim3((unsigned)a.N),
                           dim3(kTailThreads), 0, stream, a, w);
      }
    }
    // Also with no token: every row is the fill value.
    hipLaunchKernelGGL(tails_worst_sort_kernel, dim3(3), dim3(kWorstSortThreads), 0, stream, a, w);
  } else {
    launch_select<kWorstT>(a, w, stream);
  }
  return hipGetLastError();
}

}  // namespace lp
