// Correction consumers of the rollout/trainer logprobs: per-token importance
// weights of the correction ratio r = pi_train / pi_rollout with truncation
// (TIS) and an accepted interval (MIS), and sequence-level rejection by the
// accumulated K1 or K3 estimate of log r.
//
// "Rollout-Training Mismatch in LLM RL", section 2.1 (Eq. 2 and the TIS / MIS
// definitions after Eq. 3): w_TIS = min(w, C), w_MIS = w 1[l <= w <= u].
// "Diagnosing Training Inference Mismatch ...", result 5 and the discussion of
// how TIS works: the correction ratio is the old trainer probability over the
// rollout probability of the sampled token; token TIS clamps exp(log r) at C;
// sequence rejection filters a trajectory by sum_t K1(r_t) or sum_t K3(r_t);
// padding tokens get weight zero.
//
// One workgroup per sequence. Pass 1 forms the sequence statistic and the
// interval / cap counts (a fixed per-thread order, then a fixed tree), the
// workgroup decides acceptance, and pass 2 writes the weights: a rejected
// sequence's are zeros, written without reading the row again; an accepted
// sequence's re-read the row (L2 hits). For |d| < 1/64 (the usual size of a
// rollout/trainer gap) the K3 term and the weight come from one fp64 series,
// e^d - 1 - d = d^2 sum_k d^k / (k + 2)!, instead of the library's expm1 and
// exp.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lp_internal.h"

namespace lp {
namespace {

constexpr int kCorrThreads = kRowThreads;
constexpr int kCorrWaves = kCorrThreads / 64;

struct CorrPart {
  double stat, sum_w;
  int32_t valid, nonfinite, kept, capped;
};

__device__ __forceinline__ bool fin(float x) { return __builtin_isfinite(x); }

// e^d - 1 - d for |d| < 1/64: d^2 g(d), g(d) = sum_k d^k / (k + 2)! to
// d^7 / 9! (the first term left out is below 1e-17 of the sum).
__device__ __forceinline__ double k3_small(double d) {
  double g = 1.0 / 362880.0;
  g = fma(g, d, 1.0 / 40320.0);
  g = fma(g, d, 1.0 / 5040.0);
  g = fma(g, d, 1.0 / 720.0);
  g = fma(g, d, 1.0 / 120.0);
  g = fma(g, d, 1.0 / 24.0);
  g = fma(g, d, 1.0 / 6.0);
  g = fma(g, d, 0.5);
  return (d * d) * g;
}
constexpr double kSmallD = 1.0 / 64.0;

// K1(r) = -log r and K3(r) = r - 1 - log r, with log r = d.
__device__ __forceinline__ double k_term(int kind, double d) {
  if (kind == LP_REJECT_K1) return -d;
  if (kind == LP_REJECT_K3) return fabs(d) < kSmallD ? k3_small(d) : expm1(d) - d;
  return 0.0;
}

// e^d (the weight before the cap).
__device__ __forceinline__ double exp_d(double d) {
  return fabs(d) < kSmallD ? 1.0 + (d + k3_small(d)) : exp(d);
}

// Fixed XOR butterfly within the wave (DPP, ds_swizzle and readlane), then
// the waves in index order.
__device__ CorrPart block_sum(CorrPart p, CorrPart* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  p.stat = wave_sum(p.stat);
  p.sum_w = wave_sum(p.sum_w);
  p.valid = wave_sum(p.valid);
  p.nonfinite = wave_sum(p.nonfinite);
  p.kept = wave_sum(p.kept);
  p.capped = wave_sum(p.capped);
  if (lane == 0) lds[wave] = p;
  __syncthreads();
  CorrPart s = lds[0];
#pragma unroll
  for (int w = 1; w < kCorrWaves; ++w) {
    s.stat += lds[w].stat;
    s.sum_w += lds[w].sum_w;
    s.valid += lds[w].valid;
    s.nonfinite += lds[w].nonfinite;
    s.kept += lds[w].kept;
    s.capped += lds[w].capped;
  }
  __syncthreads();
  return s;
}

// Positions of thread tid in a row: groups of four consecutive positions
// 4 tid + 1024 k (one 16-byte load per array on the vector path).
template <bool kVec>
__device__ __forceinline__ void load4(const CorrectArgs& a, const float* R, const float* Tr,
                                      const uint8_t* M, int64_t i, float r[4], float t[4],
                                      bool act[4]) {
  if (kVec && i + 4 <= a.L) {
    const float4 rv = *reinterpret_cast<const float4*>(R + i);
    const float4 tv = *reinterpret_cast<const float4*>(Tr + i);
    const uint32_t mv = *reinterpret_cast<const uint32_t*>(M + i);
    r[0] = rv.x; r[1] = rv.y; r[2] = rv.z; r[3] = rv.w;
    t[0] = tv.x; t[1] = tv.y; t[2] = tv.z; t[3] = tv.w;
#pragma unroll
    for (int k = 0; k < 4; ++k) act[k] = ((mv >> (8 * k)) & 255u) != 0;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      act[k] = i + k < a.L && M[i + k] != 0;
      r[k] = act[k] ? R[i + k] : 0.f;
      t[k] = act[k] ? Tr[i + k] : 0.f;
    }
  }
}

template <bool kVec>
__device__ __forceinline__ void store4(const CorrectArgs& a, float* W, int64_t i, const float w[4]) {
  if (kVec && i + 4 <= a.L && (a.L & 3) == 0) {
    *reinterpret_cast<float4*>(W + i) = make_float4(w[0], w[1], w[2], w[3]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i + k < a.L) W[i + k] = w[k];
  }
}

// Rows of at most kHeld x 1024 positions keep pass 1's loads in registers
// for pass 2 (kHeld groups of four positions per thread); longer rows read
// the row again.
constexpr int kHeld = 3;

template <bool kVec, bool kKeep>
__global__ __launch_bounds__(kCorrThreads) void correct_kernel(CorrectArgs a) {
  __shared__ CorrPart lds[kCorrWaves];
  const int64_t n = blockIdx.x;
  const float* R = a.rollout + n * a.ld;
  const float* Tr = a.train + n * a.ld;
  const uint8_t* M = a.mask + n * a.ld;
  const int64_t step = 4 * kCorrThreads;
  float hr[kKeep ? kHeld : 1][4], ht[kKeep ? kHeld : 1][4];
  bool hact[kKeep ? kHeld : 1][4];

  // Pass 1: the sequence statistic over the counted tokens (active, both
  // scores finite), in ascending position order per thread, and the counts
  // of the interval and cap decisions (made whether or not the sequence is
  // accepted).
  CorrPart p{0.0, 0.0, 0, 0, 0, 0};
  auto fold1 = [&](const float r[4], const float t[4], const bool act[4])
      __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!act[k]) continue;
      p.valid += 1;
      if (!fin(r[k]) || !fin(t[k])) {
        p.nonfinite += 1;
        continue;
      }
      const double d = (double)t[k] - (double)r[k];
      p.stat += k_term(a.kind, d);
      const bool inside = d >= a.log_lo && d <= a.log_hi;
      p.kept += inside ? 1 : 0;
      p.capped += (inside && d >= a.log_cap) ? 1 : 0;
    }
  };
  if (kKeep) {
#pragma unroll
    for (int g = 0; g < kHeld; ++g) {
      const int64_t i = 4 * (int64_t)threadIdx.x + g * step;
      load4<kVec>(a, R, Tr, M, i, hr[g], ht[g], hact[g]);  // past L: inactive
    }
#pragma unroll
    for (int g = 0; g < kHeld; ++g) fold1(hr[g], ht[g], hact[g]);
  } else {
    for (int64_t i = 4 * (int64_t)threadIdx.x; i < a.L; i += step) {
      float r[4], t[4];
      bool act[4];
      load4<kVec>(a, R, Tr, M, i, r, t, act);
      fold1(r, t, act);
    }
  }
  const CorrPart s1 = block_sum(p, lds);
  // An overflowing K3 term makes the statistic +inf: rejected by any finite
  // upper bound.
  const bool accepted = !(s1.stat < a.rej_lo) && !(s1.stat > a.rej_hi);

  // Pass 2: weights. Inside the interval the weight is r truncated at C
  // (evaluated as C when log r >= log C, so it never overflows there);
  // outside it, on masked or non-finite tokens and in rejected sequences, 0.
  float* W = a.weights ? a.weights + n * a.L : nullptr;
  double sum_w = 0.0;
  if (accepted) {
    CorrPart q{0.0, 0.0, 0, 0, 0, 0};
    auto fold2 = [&](int64_t i, const float r[4], const float t[4], const bool act[4])
        __attribute__((always_inline)) {
      float w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[k] = 0.f;
        if (!act[k] || !fin(r[k]) || !fin(t[k])) continue;
        const double d = (double)t[k] - (double)r[k];
        if (!(d >= a.log_lo && d <= a.log_hi)) continue;
        w[k] = (float)(d >= a.log_cap ? a.cap : exp_d(d));
        q.sum_w += (double)w[k];
      }
      if (W && i < a.L) store4<kVec>(a, W, i, w);
    };
    if (kKeep) {
#pragma unroll
      for (int g = 0; g < kHeld; ++g) fold2(4 * (int64_t)threadIdx.x + g * step, hr[g], ht[g], hact[g]);
    } else {
      for (int64_t i = 4 * (int64_t)threadIdx.x; i < a.L; i += step) {
        float r[4], t[4];
        bool act[4];
        load4<kVec>(a, R, Tr, M, i, r, t, act);
        fold2(i, r, t, act);
      }
    }
    sum_w = block_sum(q, lds).sum_w;
  } else if (W) {
    const float z[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = 4 * (int64_t)threadIdx.x; i < a.L; i += step) store4<kVec>(a, W, i, z);
  }
  if (threadIdx.x == 0) {
    lp_corr_seq o;
    o.valid = s1.valid;
    o.nonfinite = s1.nonfinite;
    o.kept = s1.kept;
    o.capped = s1.capped;
    o.accepted = accepted ? 1 : 0;
    o.reserved = 0;
    o.stat = s1.stat;
    o.sum_weight = sum_w;
    a.out[n] = o;
  }
}

}  // namespace

hipError_t launch_correct(const CorrectArgs& a, hipStream_t stream) {
  const dim3 g((unsigned)a.N), b(kCorrThreads);
  const bool keep = a.L <= (int64_t)kHeld * 4 * kCorrThreads;
  if (a.vec) {
    if (keep) hipLaunchKernelGGL((correct_kernel<true, true>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((correct_kernel<true, false>), g, b, 0, stream, a);
  } else {
    if (keep) hipLaunchKernelGGL((correct_kernel<false, true>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((correct_kernel<false, false>), g, b, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace lp
