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

}  // namespace

hipError_t launch_seq_quantiles(const QuantArgs& a, hipStream_t stream) {
  const unsigned blocks = (unsigned)(3 * ((a.N + 7) / 8) * 8);  // 24 per group of 8 sequences
  if (a.vec)
    hipLaunchKernelGGL(seq_quantile_kernel<true>, dim3(blocks), dim3(kQThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(seq_quantile_kernel<false>, dim3(blocks), dim3(kQThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lp
