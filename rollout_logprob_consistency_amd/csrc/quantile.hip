// Per-sequence quantiles of |delta| for each pair (lp_compare_quantiles): the
// p50 / p95 / p99 that the AMD blog's compare() (section "Case 1: A Changes;
// B and C Stay Close") returns for one record's response-aligned arrays --
// numpy's default ("linear") quantile over the record's counted tokens,
// which the p95 / p99 row of the blog's "Check Whether the Pattern Extends
// Across the Response" refers to.
//
// One workgroup per (sequence, pair). A key is the bit pattern of the fp64
// |delta| of a counted token (active, both scores finite); as non-negative
// doubles the keys order like unsigned integers. The six order statistics
// the three quantiles interpolate between (quantile_ranks) are selected
// exactly:
//  1. One read of the scores histograms the keys' top 16 bits. The
//     difference of two finite fp32 values is 0 or has an fp64 exponent in
//     [874, 1152] (2^-149 <= |delta| < 2^130), so those 16 bits take 4 465
//     values (bin 0 holds the key 0); a scan of the 4 465 bins gives every
//     rank its 16-bit bucket and its rank inside it.
//  2. The keys of the chosen buckets -- a few percent of the row for
//     continuous differences -- are read again and gathered in LDS, and each
//     rank is found by counting: the candidate k of the bucket with
//     #{j : c_j < k} < r <= #{j : c_j <= k}.
//  3. When the buckets hold more keys than the gather buffer (many equal or
//     near-equal differences), the remaining 48 bits are selected by 8-bit
//     radix passes over the row instead, one byte per pass.
// Every count is an integer, so the result does not depend on how the
// threads are scheduled; the interpolation is the fp64 quantile_lerp.
#include "lp_internal.h"

namespace lp {
namespace {

constexpr int kQThreads = kRowThreads;
constexpr int kQWaves = kQThreads / 64;
constexpr int kQT = 6;                  // ranks lo / hi of p50, p95, p99
constexpr uint64_t kNoKey = ~0ull;      // not counted (a real key has bit 63 clear)
constexpr int kBinsPerThread = (kKeyBuckets + kQThreads - 1) / kQThreads;  // 18
constexpr int kCand = 512;              // gathered candidates

static_assert(kQThreads * kBinsPerThread >= kKeyBuckets, "every bin belongs to a thread");

__device__ __forceinline__ uint64_t key_of(float l, float r, bool act) {
  if (!act || !__builtin_isfinite(l) || !__builtin_isfinite(r)) return kNoKey;
  return (uint64_t)__double_as_longlong(fabs((double)l - (double)r));
}

// Scores and mask of the four positions i .. i + 3 of a row (inactive past
// L): one 16-byte load per score array and a 4-byte mask load when the rows
// allow them, element loads otherwise. Raw values, so that a chunk's loads
// can be in flight while the previous chunk is processed.
struct Raw4 {
  float l[4], r[4];
  bool act[4];
};

template <bool kVec>
__device__ __forceinline__ Raw4 load4(const float* Lp, const float* Rp, const uint8_t* M,
                                      int64_t L, int64_t i) {
  Raw4 q;
  if (kVec && i + 4 <= L) {
    const float4 l = *reinterpret_cast<const float4*>(Lp + i);
    const float4 r = *reinterpret_cast<const float4*>(Rp + i);
    const uint32_t m = *reinterpret_cast<const uint32_t*>(M + i);
    q.l[0] = l.x; q.l[1] = l.y; q.l[2] = l.z; q.l[3] = l.w;
    q.r[0] = r.x; q.r[1] = r.y; q.r[2] = r.z; q.r[3] = r.w;
#pragma unroll
    for (int e = 0; e < 4; ++e) q.act[e] = ((m >> (8 * e)) & 0xFFu) != 0;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q.act[e] = i + e < L && M[i + e] != 0;
      q.l[e] = q.act[e] ? Lp[i + e] : 0.f;
      q.r[e] = q.act[e] ? Rp[i + e] : 0.f;
    }
  }
  return q;
}

__device__ __forceinline__ void keys_of(const Raw4& q, uint64_t (&k)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) k[e] = key_of(q.l[e], q.r[e], q.act[e]);
}

template <bool kVec>
__global__ __launch_bounds__(kQThreads) void seq_quantile_kernel(QuantArgs a) {
  // The 4 465-bin histogram of step 1; the 8-bit histograms of step 3 reuse it.
  __shared__ uint32_t hist[kQThreads * kBinsPerThread];
  __shared__ uint64_t cand[kCand];
  __shared__ uint32_t s_part[kQWaves];
  __shared__ uint64_t s_pre[kQT], s_val[kQT];
  __shared__ int64_t s_rank[kQT], s_r[kQT];
  __shared__ uint32_t s_bk[kQT];
  __shared__ uint32_t s_ncand, s_gather;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroups are dealt to the 8 XCDs in turn by their index, and each XCD
  // has its own L2. Index 24 g + 8 p + x takes pair p of sequence 8 g + x, so
  // the three workgroups of a sequence (each reads two of its three score
  // arrays) run on one XCD at about the same time and share the reads.
  const int64_t b = blockIdx.x;
  const int64_t n = 8 * (b / 24) + (b % 8);
  const int p = (int)((b % 24) / 8);  // pair: 0 (A,B), 1 (B,C), 2 (A,C)
  if (n >= a.N) return;
  const float* Lp = (p == 1 ? a.B : a.A) + n * a.ld;
  const float* Rp = (p == 0 ? a.B : a.C) + n * a.ld;
  const uint8_t* M = a.mask + n * a.ld;
  double* out = a.out + ((size_t)n * 3 + (size_t)p) * 3;
  // Every thread takes the same number of steps over the row (four
  // consecutive positions each), so whole waves reach the ballots; positions
  // past L hold no key.
  constexpr int64_t kStep = 4 * kQThreads;
  const int64_t Lw = (a.L + kStep - 1) / kStep * kStep;

  for (int i = tid; i < kQThreads * kBinsPerThread; i += kQThreads) hist[i] = 0u;
  if (tid == 0) {
    s_ncand = 0u;
    s_gather = 0u;
  }
  __syncthreads();

  // Each walk over the row keeps the next chunk's loads in flight while it
  // processes the current one (the last chunk is loaded twice rather than
  // branching); `visit` sees the four keys of every position of the row.
  auto walk = [&](auto&& visit) {
    Raw4 q = load4<kVec>(Lp, Rp, M, a.L, 4 * tid);
    for (int64_t i = 4 * tid; i < Lw; i += kStep) {
      const Raw4 nq = load4<kVec>(Lp, Rp, M, a.L, min(i + kStep, Lw - kStep + 4 * tid));
      uint64_t k[4];
      keys_of(q, k);
      visit(k);
      q = nq;
    }
  };

  // Step 1: the 16-bit bucket histogram.
  walk([&](const uint64_t (&k)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) wave_hist_add(hist, key_bucket(k[e]), k[e] != kNoKey, lane);
  });
  __syncthreads();
  // Thread j owns bins [18 j, 18 j + 18): their sum, an exclusive scan of the
  // sums over the threads (the count is the last inclusive value).
  const int b0 = tid * kBinsPerThread;
  uint32_t mine = 0u;
#pragma unroll
  for (int b = 0; b < kBinsPerThread; ++b) mine += hist[b0 + b];
  uint32_t incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_part[wave] = incl;
  __syncthreads();
  uint32_t before = 0u, count32 = 0u;
#pragma unroll
  for (int v = 0; v < kQWaves; ++v) {
    before += v < wave ? s_part[v] : 0u;
    count32 += s_part[v];
  }
  const int64_t count = count32;
  if (count == 0) {
    if (tid < 3) out[tid] = 0.0;
    return;
  }
  const int64_t excl = (int64_t)before + incl - mine;
  // The six ranks, once per workgroup.
  if (tid < kQT) {
    int64_t lo, hi;
    quantile_ranks(count, quantile_prob(tid >> 1), &lo, &hi);
    s_r[tid] = (tid & 1) ? hi : lo;
  }
  __syncthreads();
  // The thread whose bins hold rank r finds the bucket and the rank within.
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    const int64_t r = s_r[t];
    if (excl < r && r <= excl + mine) {
      int64_t below = excl;
      int b = 0;
      while (below + (int64_t)hist[b0 + b] < r) below += hist[b0 + b++];
      const uint32_t bk = (uint32_t)(b0 + b);
      // Bucket 0 holds only the key 0: that rank is settled.
      s_pre[t] = bk == 0 ? 0ull : (uint64_t)(bk - 1u + kKeyTop16Lo);
      s_rank[t] = bk == 0 ? 0 : r - below;
      s_bk[t] = bk;
      s_val[t] = 0ull;
    }
  }
  __syncthreads();
  // The chosen buckets' keys, each distinct bucket counted once.
  if (tid == 0) {
    uint32_t nc = 0u;
    for (int t = 0; t < kQT; ++t) {
      bool first = s_bk[t] != 0u;
      for (int u = 0; u < t; ++u) first = first && s_bk[u] != s_bk[t];
      if (first) nc += hist[s_bk[t]];
    }
    s_ncand = nc;
  }
  __syncthreads();
  const bool gather = s_ncand <= (uint32_t)kCand;
  uint64_t pre[kQT];
  bool live[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    pre[t] = s_pre[t];
    live[t] = s_rank[t] > 0;
  }

  if (gather) {
    // Step 2: gather the chosen buckets' keys, then rank by counting.
    walk([&](const uint64_t (&kk)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t k = kk[e];
        bool m = false;
#pragma unroll
        for (int t = 0; t < kQT; ++t) m = m || (live[t] && k != kNoKey && (k >> 48) == pre[t]);
        const uint64_t mb = __ballot(m);
        if (mb == 0) continue;
        const int first = __ffsll((long long)mb) - 1;
        uint32_t base = 0u;
        if (lane == first) base = atomicAdd(&s_gather, (uint32_t)__popcll(mb));
        base = (uint32_t)__shfl((int)base, first);
        if (m) cand[base + (uint32_t)__popcll(mb & ((1ull << lane) - 1ull))] = k;
      }
    });
    __syncthreads();
    const int nc = (int)s_gather;
    for (int i = tid; i < nc; i += kQThreads) {
      const uint64_t k = cand[i];
      const uint64_t top = k >> 48;
      int32_t less = 0, leq = 0;
#pragma unroll 8
      for (int j = 0; j < nc; ++j) {
        const uint64_t c = cand[j];
        const bool same = (c >> 48) == top;
        less += (same && c < k) ? 1 : 0;
        leq += (same && c <= k) ? 1 : 0;
      }
#pragma unroll
      for (int t = 0; t < kQT; ++t)
        if (live[t] && top == pre[t] && less < s_rank[t] && s_rank[t] <= leq) s_val[t] = k;
    }
    __syncthreads();
  } else {
    // Step 3: 8-bit radix passes over the remaining 48 bits, from the row.
    uint32_t (*h8)[256] = reinterpret_cast<uint32_t (*)[256]>(hist);
    for (int pass = 2; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      int src[kQT];
      bool use[kQT];
      bool any = false;
#pragma unroll
      for (int t = 0; t < kQT; ++t) {
        pre[t] = s_pre[t];
        live[t] = s_rank[t] > 0;
      }
#pragma unroll
      for (int t = 0; t < kQT; ++t) {
        src[t] = t;
        for (int u = 0; u < t; ++u)
          if (live[u] && pre[u] == pre[t]) {
            src[t] = u;
            break;
          }
        use[t] = live[t] && src[t] == t;
        any = any || live[t];
      }
      if (!any) break;  // uniform: from LDS after a barrier
      for (int i = tid; i < kQT * 256; i += kQThreads) (&h8[0][0])[i] = 0u;
      __syncthreads();
      walk([&](const uint64_t (&kk)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint64_t k = kk[e];
          const uint32_t digit = (uint32_t)(k >> shift) & 255u;
#pragma unroll
          for (int t = 0; t < kQT; ++t) {
            if (!use[t]) continue;  // uniform
            wave_hist_add(h8[t], digit, k != kNoKey && (k >> (shift + 8)) == pre[t], lane);
          }
        }
      });
      __syncthreads();
      for (int t = wave; t < kQT; t += kQWaves) {
        const int64_t rank = s_rank[t];
        if (rank <= 0) continue;  // uniform within the wave
        uint32_t c[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = h8[src[t]][4 * lane + k];
        const uint32_t lsum = c[0] + c[1] + c[2] + c[3];
        uint32_t inc = lsum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = (uint32_t)__shfl_up((int)inc, off);
          if (lane >= off) inc += o;
        }
        const int64_t ex = (int64_t)inc - lsum;
        if (ex < rank && rank <= (int64_t)inc) {
          int64_t below = ex;
          int k = 0;
          while (below + (int64_t)c[k] < rank) below += c[k++];
          s_pre[t] = (pre[t] << 8) | (uint64_t)(4 * lane + k);
          s_rank[t] = rank - below;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < kQT; ++t)
      if (tid == t && s_rank[t] > 0) s_val[t] = s_pre[t];  // the full key
    __syncthreads();
  }
  if (tid < 3) {
    const double lo = __longlong_as_double((long long)s_val[2 * tid]);
    const double hi = __longlong_as_double((long long)s_val[2 * tid + 1]);
    out[tid] = quantile_lerp(count, quantile_prob(tid), lo, hi);
  }
}

// ---------------------------------------------------------------------------
// Rows of at most 3 072 positions: one wave per (sequence, pair) holding the
// row's keys in registers (kJ chunks of four positions per lane), so the row
// is read once and no step waits for another wave.
//  1. A histogram of 4 096 buckets: the key 0; the keys whose top 16 bits
//     are under kWLo (below 1.125 * 2^-126) together; one bucket per top-16
//     value from kWLo up.
//     Its scan gives each rank a key range and the rank inside that range.
//  2. While a range holds more than kWGroup keys (many equal or near-equal
//     differences), a histogram of the next 12 bits below the range's common
//     prefix narrows it; a range narrowed to one key value is settled.
//  3. The keys of the remaining ranges are gathered in LDS, grouped by range,
//     and each rank is found by counting within its group: the key c with
//     #{keys < c} < rank <= #{keys <= c}.
// All counts are integers, so the selected keys are exact and the result
// does not depend on scheduling; the same fp64 quantile_lerp follows.
// ---------------------------------------------------------------------------
constexpr int kWBins = 4096;                           // 16-bit counters, two per word
constexpr uint32_t kWLo = kKeyTop16Hi - (kWBins - 3);  // top-16 value of bucket 2
constexpr int kWGroup = 64;                            // ranges up to this size are counted
constexpr int kWMaxJ = 9;                              // 9 x 256 = 2 304 positions

// Bucket of a non-zero counted key (bucket 0, the key 0, is counted apart).
__device__ __forceinline__ uint32_t wbucket_nz(uint64_t k) {
  const uint32_t t = (uint32_t)(k >> 48);  // at most kKeyTop16Hi for a finite difference
  return max(t, kWLo - 1u) - (kWLo - 2u);
}

// Inclusive prefix sum over the wave's lanes on DPP: shifts by 1, 2, 4 and 8
// inside each row of 16 (lanes with no source add 0), then the last lane of
// row 0 (and 2) is broadcast into row 1 (and 3), and the last lane of row 1
// into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Lane l owns bins [64 l, 64 l + 64) of the 16-bit histogram (words
// [32 l, 32 l + 32)); `mine` is their sum and the result its inclusive
// prefix over the lanes. The lanes start at different 16-byte chunks of
// their 128 bytes, which spreads the reads over the LDS banks.
__device__ __forceinline__ uint32_t hist_prefix(const uint32_t* h, int lane, uint32_t& mine) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint4* h4 = reinterpret_cast<const uint4*>(h) + 8 * lane;
  uint32_t s = 0u;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint4 v = h4[(w + lane) & 7];
    const u16x2 one = {1, 1};
    s = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, v.x), one, s, false);
    s = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, v.y), one, s, false);
    s = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, v.z), one, s, false);
    s = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, v.w), one, s, false);
  }
  mine = s;
  return wave_incl_scan(s);
}

// The bin of the r-th counted key (1 <= r <= total); `below` keys lie in
// lower bins and `cnt` in this one. r is wave-uniform.
__device__ __forceinline__ uint32_t hist_find(const uint32_t* h, int lane, uint32_t incl,
                                              uint32_t mine, uint32_t r, uint32_t& below,
                                              uint32_t& cnt) {
  const int o = __ffsll((long long)__ballot(incl >= r)) - 1;  // lane holding the bin
  const uint32_t ex = (uint32_t)__builtin_amdgcn_readlane((int)(incl - mine), o);
  const uint32_t bin = 64u * (uint32_t)o + (uint32_t)lane;
  const uint32_t c = (h[bin >> 1] >> ((bin & 1u) << 4)) & 0xFFFFu;
  const uint32_t inc = wave_incl_scan(c);
  const int j = __ffsll((long long)__ballot(ex + inc >= r)) - 1;
  below = ex + (uint32_t)__builtin_amdgcn_readlane((int)(inc - c), j);
  cnt = (uint32_t)__builtin_amdgcn_readlane((int)c, j);
  return 64u * (uint32_t)o + (uint32_t)j;
}

// Lane masks of 64-bit key comparisons, formed in scalar registers (a ballot
// of a combined condition would first materialise it per lane).
__device__ __forceinline__ uint64_t mask_eq(uint64_t x, uint64_t y) {
  return __builtin_amdgcn_uicmpl(x, y, 32);  // ICMP_EQ
}
__device__ __forceinline__ uint64_t mask_ne(uint64_t x, uint64_t y) {
  return __builtin_amdgcn_uicmpl(x, y, 33);  // ICMP_NE
}
__device__ __forceinline__ uint64_t mask_in(uint64_t x, uint64_t lo, uint64_t hi) {
  return __builtin_amdgcn_uicmpl(x, lo, 35) & __builtin_amdgcn_uicmpl(x, hi, 36);  // UGE, ULT
}

template <bool kVec, int kJ>
__device__ __forceinline__ void seq_quantile_wave(const QuantArgs& a) {
  constexpr int kK = 4 * kJ;
  // The histogram (4 096 16-bit bins); afterwards the gathered keys.
  __shared__ __attribute__((aligned(16))) uint32_t h[kWBins / 2];
  uint64_t* cand = reinterpret_cast<uint64_t*>(h);
  static_assert(kQT * kWGroup * sizeof(uint64_t) <= sizeof(h), "candidates fit");
  const int lane = threadIdx.x;
  // Same placement as the workgroup kernel: index 24 g + 8 p + x takes pair p
  // of sequence 8 g + x, so a sequence's three waves share its rows in L2.
  const int64_t b = blockIdx.x;
  const int64_t n = 8 * (b / 24) + (b % 8);
  const int p = (int)((b % 24) / 8);
  if (n >= a.N) return;
  const float* Lp = (p == 1 ? a.B : a.A) + n * a.ld;
  const float* Rp = (p == 0 ? a.B : a.C) + n * a.ld;
  const uint8_t* M = a.mask + n * a.ld;
  double* out = a.out + ((size_t)n * 3 + (size_t)p) * 3;
  const uint32_t L = (uint32_t)a.L;
  // Range-checked buffer loads: positions past the row read as zeros and are
  // not counted, so the last chunk needs no branch (the vector form runs only
  // on rows of a multiple of 4 positions: see launch_wave).
  const __amdgpu_buffer_rsrc_t lr = row_rsrc(Lp, 4u * L), rr = row_rsrc(Rp, 4u * L);
  const __amdgpu_buffer_rsrc_t mr = row_rsrc(M, L);

  uint4* h4 = reinterpret_cast<uint4*>(h);
  auto zero_hist = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) h4[64 * i + lane] = make_uint4(0u, 0u, 0u, 0u);
  };
  zero_hist();

  // Every chunk's loads are issued before any key is formed. The mask bytes
  // of a chunk stay packed in one word (byte e: position i + e).
  float lv[kK], rv[kK];
  uint32_t mw[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const uint32_t i = 256u * (uint32_t)j + 4u * (uint32_t)lane;
    if (kVec) {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 l4 = __builtin_amdgcn_raw_buffer_load_b128(lr, 4u * i, 0, 0);
      const u32x4 r4 = __builtin_amdgcn_raw_buffer_load_b128(rr, 4u * i, 0, 0);
      mw[j] = __builtin_amdgcn_raw_buffer_load_b32(mr, i, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lv[4 * j + e] = __uint_as_float(l4[e]);
        rv[4 * j + e] = __uint_as_float(r4[e]);
      }
    } else {
      mw[j] = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lv[4 * j + e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lr, 4u * (i + e), 0, 0));
        rv[4 * j + e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, 4u * (i + e), 0, 0));
        mw[j] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(mr, i + e, 0, 0) << (8 * e);
      }
    }
  }
  // Keys: the fp64 difference is finite exactly when both scores are.
  uint64_t k[kK];
#pragma unroll
  for (int j = 0; j < kJ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = 256u * (uint32_t)j + 4u * (uint32_t)lane + (uint32_t)e;
      const double dl = (double)lv[4 * j + e] - (double)rv[4 * j + e];
      const bool ok = i < L && ((mw[j] >> (8 * e)) & 0xFFu) != 0u && __builtin_isfinite(dl);
      k[4 * j + e] = ok ? (uint64_t)__double_as_longlong(fabs(dl)) : kNoKey;
    }

  // Step 1. Zero differences (identical scores, often most of a row) are
  // counted with ballots; every other counted key adds 1 to its 16-bit bin.
  __syncthreads();
  uint32_t zeros = 0u;
#pragma unroll
  for (int e = 0; e < kK; ++e) {
    zeros += (uint32_t)__popcll(mask_eq(k[e], 0ull));
    const uint64_t hm = mask_ne(k[e], 0ull) & mask_ne(k[e], kNoKey);
    if (hm == 0) continue;
    if (__builtin_amdgcn_inverse_ballot_w64(hm)) {
      const uint32_t bin = wbucket_nz(k[e]);
      atomicAdd(&h[bin >> 1], 1u << ((bin & 1u) << 4));
    }
  }
  if (lane == 0) atomicAdd(&h[0], zeros);  // bin 0: the low half of word 0
  __syncthreads();
  uint32_t mine;
  const uint32_t incl = hist_prefix(h, lane, mine);
  const uint32_t count = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  if (count == 0u) {
    if (lane < 3) out[lane] = 0.0;
    return;
  }
  // Per rank (wave-uniform): its key range [lo, hi), the bit above which
  // every key of the range agrees (64: none), its rank and size there. A
  // range settled on one key value has sh == 0, and lo is that key.
  uint64_t lo[kQT], hi[kQT];
  int sh[kQT];
  uint32_t rk[kQT], m[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    int64_t rl, rh;
    quantile_ranks((int64_t)count, quantile_prob(t >> 1), &rl, &rh);
    uint32_t below, cnt;
    const uint32_t bk = hist_find(h, lane, incl, mine, (uint32_t)((t & 1) ? rh : rl), below, cnt);
    rk[t] = (uint32_t)((t & 1) ? rh : rl) - below;
    m[t] = cnt;
    if (bk == 0u) {
      lo[t] = hi[t] = 0ull;
      sh[t] = 0;
    } else if (bk == 1u) {
      lo[t] = 1ull;
      hi[t] = (uint64_t)kWLo << 48;
      sh[t] = 64;
    } else {
      const uint64_t top = (uint64_t)(bk - 2u + kWLo);
      lo[t] = top << 48;
      hi[t] = (top + 1ull) << 48;
      sh[t] = 48;
    }
  }

  // Step 2: each pass narrows every rank that shares the first oversized
  // range by 12 bits (or to its last bits), so at most 6 passes per range.
  for (int pass = 0; pass < 6 * kQT; ++pass) {
    int t0 = -1;
#pragma unroll
    for (int t = 0; t < kQT; ++t)
      if (t0 < 0 && sh[t] != 0 && m[t] > (uint32_t)kWGroup) t0 = t;
    if (t0 < 0) break;
    uint64_t rlo = 0ull, rhi = 0ull;
    int rsh = 0;
#pragma unroll
    for (int t = 0; t < kQT; ++t)
      if (t == t0) {
        rlo = lo[t];
        rhi = hi[t];
        rsh = sh[t];
      }
    const int ds = rsh > 12 ? rsh - 12 : 0;
    const uint32_t dmask = (1u << (rsh - ds)) - 1u;  // the bits in [ds, rsh): 12, or 4 at the end
    const uint64_t base = rsh >= 64 ? 0ull : (rlo >> rsh) << rsh;
    __syncthreads();  // the previous scan's reads are done
    zero_hist();
    __syncthreads();
    // The keys of a crowded range often share a bin: when every key of the
    // wave in the range does, one lane adds them all.
#pragma unroll
    for (int e = 0; e < kK; ++e) {
      const uint64_t hm = mask_in(k[e], rlo, rhi);
      if (hm == 0) continue;
      const uint32_t bin = (uint32_t)(k[e] >> ds) & dmask;
      const int first = __ffsll((long long)hm) - 1;
      const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
      if ((hm & __builtin_amdgcn_uicmp(bin, b0, 32)) == hm) {
        if (lane == first) atomicAdd(&h[b0 >> 1], (uint32_t)__popcll(hm) << ((b0 & 1u) << 4));
      } else if (__builtin_amdgcn_inverse_ballot_w64(hm)) {
        atomicAdd(&h[bin >> 1], 1u << ((bin & 1u) << 4));
      }
    }
    __syncthreads();
    uint32_t mine2;
    const uint32_t incl2 = hist_prefix(h, lane, mine2);
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      if (sh[t] == 0 || lo[t] != rlo || hi[t] != rhi) continue;
      uint32_t below, cnt;
      const uint32_t bin = hist_find(h, lane, incl2, mine2, rk[t], below, cnt);
      const uint64_t sub = base + ((uint64_t)bin << ds);
      lo[t] = sub > rlo ? sub : rlo;
      hi[t] = sub + (1ull << ds) < rhi ? sub + (1ull << ds) : rhi;
      sh[t] = ds;
      rk[t] -= below;
      m[t] = cnt;
    }
  }

  // Step 3: groups of equal ranges, in target order; g[t] = the first target
  // of t's group.
  int g[kQT];
  uint32_t goff[kQT];
  uint32_t nc = 0u, maxm = 0u;
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    g[t] = t;
#pragma unroll
    for (int u = 0; u < t; ++u)
      if (g[t] == t && sh[u] != 0 && lo[u] == lo[t] && hi[u] == hi[t]) g[t] = u;
    goff[t] = nc;
    if (sh[t] != 0 && g[t] == t) {
      nc += m[t];
      maxm = m[t] > maxm ? m[t] : maxm;
    }
  }
  // The group structure is fixed before any rank is settled below.
  bool open3[kQT], ldr[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    open3[t] = sh[t] != 0;
    ldr[t] = open3[t] && g[t] == t;
  }
  if (nc > 0u) {
    __syncthreads();  // the last scan's reads of the histogram are done
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      if (!ldr[t]) continue;
      uint32_t off = goff[t];
#pragma unroll
      for (int e = 0; e < kK; ++e) {
        const uint64_t mb = mask_in(k[e], lo[t], hi[t]);
        if (mb == 0) continue;
        if (__builtin_amdgcn_inverse_ballot_w64(mb)) cand[off + lanes_below(mb)] = k[e];
        off += (uint32_t)__popcll(mb);
      }
    }
    __syncthreads();
    for (uint32_t c0 = 0u; c0 < nc; c0 += 64u) {
      const uint32_t i = c0 + (uint32_t)lane;
      const bool has = i < nc;
      // This candidate's group: the last group starting at or below i.
      int mg = -1;
      uint32_t moff = 0u, mm = 0u;
#pragma unroll
      for (int t = 0; t < kQT; ++t)
        if (ldr[t] && goff[t] <= i) {
          mg = t;
          moff = goff[t];
          mm = m[t];
        }
      const uint64_t c = has ? cand[i] : 0ull;
      uint32_t less = 0u, leq = 0u;
      for (uint32_t j = 0u; j < maxm; ++j) {
        const uint64_t cj = cand[moff + j];  // below nc + 64: inside the array
        const bool v = has && j < mm;
        less += (v && cj < c) ? 1u : 0u;
        leq += (v && cj <= c) ? 1u : 0u;
      }
      // A rank's key (equal keys may answer it in several rounds: the same
      // value) replaces the range's lower end, which the rounds no longer read.
#pragma unroll
      for (int t = 0; t < kQT; ++t) {
        if (!open3[t]) continue;
        const uint64_t hb = __ballot(has && mg == g[t] && less < rk[t] && rk[t] <= leq);
        if (hb == 0) continue;
        const int src = __ffsll((long long)hb) - 1;
        const uint32_t vlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c, src);
        const uint32_t vhi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(c >> 32), src);
        lo[t] = ((uint64_t)vhi << 32) | vlo;
      }
    }
  }
  if (lane < 3) {
    uint64_t vl = lo[0], vh = lo[1];
#pragma unroll
    for (int q = 1; q < 3; ++q)
      if (lane == q) {
        vl = lo[2 * q];
        vh = lo[2 * q + 1];
      }
    out[lane] = quantile_lerp((int64_t)count, quantile_prob(lane),
                              __longlong_as_double((long long)vl), __longlong_as_double((long long)vh));
  }
}

// Rows with 16-byte loads: at most 96 VGPRs, so 5 waves share a SIMD (at the
// compiler's own choice of 100 it would be 4; the selection is issue-bound).
// The element-load form keeps its registers (capped, it would spill).
template <int kJ>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(5))) void seq_quantile_wave_kernel(
    QuantArgs a) {
  seq_quantile_wave<true, kJ>(a);
}

template <int kJ>
__global__ __launch_bounds__(64) void seq_quantile_wave_elem_kernel(QuantArgs a) {
  seq_quantile_wave<false, kJ>(a);
}

// Rows of 2 305 to 3 072 positions: 12 chunks of keys per lane, with no
// register cap (the keys alone take 96 VGPRs; 129 in all, 3 waves per SIMD).
// With 16 chunks (rows up to 4 096) the wave form ran slower than the
// workgroup kernel at 2 waves per SIMD, so longer rows take that kernel.
template <bool kVec, int kJ>
__global__ __launch_bounds__(64) void seq_quantile_wave_long_kernel(QuantArgs a) {
  seq_quantile_wave<kVec, kJ>(a);
}

template <int kJ>
void launch_wave_long(const QuantArgs& a, unsigned blocks, hipStream_t stream) {
  if (a.vec && (a.L & 3) == 0)
    hipLaunchKernelGGL((seq_quantile_wave_long_kernel<true, kJ>), dim3(blocks), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((seq_quantile_wave_long_kernel<false, kJ>), dim3(blocks), dim3(64), 0, stream, a);
}

// A 16-byte buffer load that reaches past the resource's end returns zeros
// as a whole (not per dword), so rows take the vector loads only when every
// group of four positions lies inside the row.
template <int kJ>
void launch_wave(const QuantArgs& a, unsigned blocks, hipStream_t stream) {
  if (a.vec && (a.L & 3) == 0)
    hipLaunchKernelGGL((seq_quantile_wave_kernel<kJ>), dim3(blocks), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((seq_quantile_wave_elem_kernel<kJ>), dim3(blocks), dim3(64), 0, stream, a);
}

}  // namespace

hipError_t launch_seq_quantiles(const QuantArgs& a, hipStream_t stream) {
  const unsigned blocks = (unsigned)(3 * ((a.N + 7) / 8) * 8);  // 24 per group of 8 sequences
  if (a.L <= 256 * 3) launch_wave<3>(a, blocks, stream);
  else if (a.L <= 256 * 6) launch_wave<6>(a, blocks, stream);
  else if (a.L <= 256 * kWMaxJ) launch_wave<kWMaxJ>(a, blocks, stream);
  else if (a.L <= 256 * 12) launch_wave_long<12>(a, blocks, stream);
  else if (a.vec)
    hipLaunchKernelGGL(seq_quantile_kernel<true>, dim3(blocks), dim3(kQThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(seq_quantile_kernel<false>, dim3(blocks), dim3(kQThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lp
