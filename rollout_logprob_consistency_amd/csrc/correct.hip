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
// One workgroup per sequence. Pass 1 forms the sequence statistic (a fixed
// per-thread order, then a fixed tree), the workgroup decides acceptance,
// pass 2 writes the weights (its reads of the row hit in L2).
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

// K1(r) = -log r and K3(r) = r - 1 - log r, with log r = d.
__device__ __forceinline__ double k_term(int kind, double d) {
  if (kind == LP_REJECT_K1) return -d;
  if (kind == LP_REJECT_K3) return expm1(d) - d;
  return 0.0;
}

// Fixed XOR butterfly within the wave, then waves in index order.
__device__ CorrPart block_sum(CorrPart p, CorrPart* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    p.stat += __shfl_xor(p.stat, off);
    p.sum_w += __shfl_xor(p.sum_w, off);
    p.valid += __shfl_xor(p.valid, off);
    p.nonfinite += __shfl_xor(p.nonfinite, off);
    p.kept += __shfl_xor(p.kept, off);
    p.capped += __shfl_xor(p.capped, off);
  }
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
__global__ __launch_bounds__(kCorrThreads) void correct_kernel(CorrectArgs a) {
  __shared__ CorrPart lds[kCorrWaves];
  const int64_t n = blockIdx.x;
  const float* R = a.rollout + n * a.ld;
  const float* Tr = a.train + n * a.ld;
  const uint8_t* M = a.mask + n * a.ld;
  const int64_t step = 4 * kCorrThreads;

  // Pass 1: the sequence statistic over the counted tokens (active, both
  // scores finite), in ascending position order per thread.
  CorrPart p{0.0, 0.0, 0, 0, 0, 0};
  for (int64_t i = 4 * (int64_t)threadIdx.x; i < a.L; i += step) {
    float r[4], t[4];
    bool act[4];
    load4<kVec>(a, R, Tr, M, i, r, t, act);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!act[k]) continue;
      p.valid += 1;
      if (!fin(r[k]) || !fin(t[k])) {
        p.nonfinite += 1;
        continue;
      }
      p.stat += k_term(a.kind, (double)t[k] - (double)r[k]);
    }
  }
  const CorrPart s1 = block_sum(p, lds);
  // An overflowing K3 term makes the statistic +inf: rejected by any finite
  // upper bound.
  const bool accepted = !(s1.stat < a.rej_lo) && !(s1.stat > a.rej_hi);

  // Pass 2: weights. Inside the interval the weight is r truncated at C
  // (evaluated as C when log r >= log C, so it never overflows there);
  // outside it, on masked or non-finite tokens and in rejected sequences, 0.
  CorrPart q{0.0, 0.0, 0, 0, 0, 0};
  float* W = a.weights ? a.weights + n * a.L : nullptr;
  for (int64_t i = 4 * (int64_t)threadIdx.x; i < a.L; i += step) {
    float r[4], t[4], w[4];
    bool act[4];
    load4<kVec>(a, R, Tr, M, i, r, t, act);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w[k] = 0.f;
      if (!act[k] || !fin(r[k]) || !fin(t[k])) continue;
      const double d = (double)t[k] - (double)r[k];
      if (!(d >= a.log_lo && d <= a.log_hi)) continue;
      q.kept += 1;
      const bool cap = d >= a.log_cap;
      q.capped += cap ? 1 : 0;
      if (accepted) {
        w[k] = (float)(cap ? a.cap : exp(d));
        q.sum_w += (double)w[k];
      }
    }
    if (W) {
      if (kVec && i + 4 <= a.L && (a.L & 3) == 0) {
        *reinterpret_cast<float4*>(W + i) = make_float4(w[0], w[1], w[2], w[3]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (i + k < a.L) W[i + k] = w[k];
      }
    }
  }
  const CorrPart s2 = block_sum(q, lds);
  if (threadIdx.x == 0) {
    lp_corr_seq o;
    o.valid = s1.valid;
    o.nonfinite = s1.nonfinite;
    o.kept = s2.kept;
    o.capped = s2.capped;
    o.accepted = accepted ? 1 : 0;
    o.reserved = 0;
    o.stat = s1.stat;
    o.sum_weight = s2.sum_w;
    a.out[n] = o;
  }
}

}  // namespace

hipError_t launch_correct(const CorrectArgs& a, hipStream_t stream) {
  if (a.vec)
    hipLaunchKernelGGL(correct_kernel<true>, dim3((unsigned)a.N), dim3(kCorrThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(correct_kernel<false>, dim3((unsigned)a.N), dim3(kCorrThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lp
