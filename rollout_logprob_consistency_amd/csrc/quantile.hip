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
// the three quantiles interpolate between (quantile_ranks) are found by an
// 8-pass MSD radix selection, one byte per pass: LDS histograms, the
// selection inside the workgroup, nothing in global memory but the inputs
// and the output. Ranks whose selected prefixes agree share one histogram
// (all six in pass 0). Rows of up to kCache positions keep their keys in LDS
// after the first read; longer rows recompute them from the scores in every
// pass. Every count is an integer, so the result does not depend on how the
// threads are scheduled, and the interpolation is the fp64 quantile_lerp.
#include "lp_internal.h"

namespace lp {
namespace {

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / 64;
constexpr int kCache = 4096;           // keys kept in LDS (32 KiB)
constexpr int kQT = 6;                 // ranks lo / hi of p50, p95, p99
constexpr uint64_t kNoKey = ~0ull;     // not counted (a real key has bit 63 clear)

__device__ __forceinline__ uint64_t key_of(float l, float r, bool act) {
  if (!act || !__builtin_isfinite(l) || !__builtin_isfinite(r)) return kNoKey;
  return (uint64_t)__double_as_longlong(fabs((double)l - (double)r));
}

__global__ __launch_bounds__(kQThreads) void seq_quantile_kernel(QuantArgs a) {
  __shared__ uint64_t keys[kCache];
  __shared__ uint32_t hist[kQT][256];
  __shared__ uint64_t s_pre[kQT];
  __shared__ int64_t s_rank[kQT];
  __shared__ uint32_t s_part[kQWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = blockIdx.x;
  const int p = blockIdx.y;  // pair: 0 (A,B), 1 (B,C), 2 (A,C)
  const float* Lp = (p == 1 ? a.B : a.A) + n * a.ld;
  const float* Rp = (p == 0 ? a.B : a.C) + n * a.ld;
  const uint8_t* M = a.mask + n * a.ld;
  const bool cached = a.L <= kCache;

  // First read: keys (into LDS when the row fits) and the count.
  uint32_t mine = 0u;
  for (int64_t i = tid; i < a.L; i += kQThreads) {
    const uint64_t k = key_of(Lp[i], Rp[i], M[i] != 0);
    if (cached) keys[i] = k;
    mine += k != kNoKey ? 1u : 0u;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mine += (uint32_t)__shfl_xor((int)mine, off);
  if (lane == 0) s_part[wave] = mine;
  __syncthreads();
  int64_t count = 0;
#pragma unroll
  for (int v = 0; v < kQWaves; ++v) count += s_part[v];
  double* out = a.out + ((size_t)p * (size_t)a.N + (size_t)n) * 3;
  if (count == 0) {
    if (tid < 3) out[tid] = 0.0;
    return;
  }
  if (tid < kQT) {
    int64_t lo, hi;
    quantile_ranks(count, quantile_prob(tid >> 1), &lo, &hi);
    s_rank[tid] = (tid & 1) ? hi : lo;
    s_pre[tid] = 0ull;
  }
  __syncthreads();

  // Every thread takes the same number of steps, so whole waves reach the
  // ballots (positions past L hold no key).
  const int64_t Lw = (a.L + kQThreads - 1) / kQThreads * kQThreads;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    uint64_t pre[kQT];
    int src[kQT];
    bool use[kQT];  // this target keeps the histogram of its prefix
    bool any = false;
#pragma unroll
    for (int t = 0; t < kQT; ++t) pre[t] = s_pre[t];
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      const bool live = s_rank[t] > 0;
      src[t] = t;
      for (int u = 0; u < t; ++u)
        if (s_rank[u] > 0 && pre[u] == pre[t]) {
          src[t] = u;
          break;
        }
      use[t] = live && src[t] == t;
      any = any || live;
    }
    if (!any) break;  // uniform: read from LDS after a barrier
    for (int i = tid; i < kQT * 256; i += kQThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < Lw; i += kQThreads) {
      const uint64_t k = i < a.L ? (cached ? keys[i] : key_of(Lp[i], Rp[i], M[i] != 0)) : kNoKey;
      const bool ok = k != kNoKey;
      const uint32_t digit = (uint32_t)(k >> shift) & 255u;
#pragma unroll
      for (int t = 0; t < kQT; ++t) {
        if (!use[t]) continue;  // uniform
        const bool hit = ok && (pass == 0 || (k >> (shift + 8)) == pre[t]);
        const uint64_t hb = __ballot(hit);
        if (hb == 0) continue;
        // One atomic for the wave when all its hits share a bin.
        const int first = __ffsll((long long)hb) - 1;
        const uint32_t d0 = (uint32_t)__shfl((int)digit, first);
        if (__ballot(hit && digit != d0) == 0) {
          if (lane == first) atomicAdd(&hist[t][d0], (uint32_t)__popcll(hb));
        } else if (hit) {
          atomicAdd(&hist[t][digit], 1u);
        }
      }
    }
    __syncthreads();
    // One wave per target in turn: the bin that holds the target's rank.
    for (int t = wave; t < kQT; t += kQWaves) {
      const int64_t rank = s_rank[t];
      if (rank <= 0) continue;  // uniform within the wave
      uint32_t c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = hist[src[t]][4 * lane + k];
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
        const uint32_t bin = 4 * lane + k;
        // A key with a zero top byte is 0: the difference of two fp32 scores
        // is 0 or at least 2^-149 in magnitude (a top byte of at least 0x36).
        s_pre[t] = (pass ? (pre[t] << 8) : 0ull) | bin;
        s_rank[t] = (pass == 0 && bin == 0) ? 0 : rank - below;
      }
    }
    __syncthreads();
  }
  if (tid < 3) {
    const double lo = __longlong_as_double((long long)s_pre[2 * tid]);
    const double hi = __longlong_as_double((long long)s_pre[2 * tid + 1]);
    out[tid] = quantile_lerp(count, quantile_prob(tid), lo, hi);
  }
}

}  // namespace

hipError_t launch_seq_quantiles(const QuantArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(seq_quantile_kernel, dim3((unsigned)a.N, 3), dim3(kQThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lp
