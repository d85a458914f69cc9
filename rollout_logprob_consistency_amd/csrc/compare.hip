// Three-way comparison of generation (A), replay (B) and trainer (C)
// logprobs on gfx950.
//
// Per sequence and per pair (A,B), (B,C), (A,C) -- the pair order and the
// left-minus-right convention of the AMD blog "Debugging Logprob Mismatches
// in LLM Reinforcement Learning" (section "Check Whether the Pattern
// Extends") -- over the masked-in tokens only:
//  * bitwise mismatch count, first mismatching active index and longest run
//    of mismatches ("Fault localization and mismatch bisect", sections
//    "Per-sequence observation patterns" and "Compare per-token logprobs");
//  * max / sum of |delta| and the signed sum ("Metric measurement basis":
//    logprob_mae; the blog's signed mean);
//  * Schulman k3 = expm1(d) - d with d = right - left, overflow counted and
//    never clipped ("Metric measurement basis"); for |d| < 0.5 the
//    exponential terms are evaluated in fp32 (k3 by its Taylor series), beyond
//    that in fp64;
//  * token and sequence truncated importance weights min(exp(d), C) and
//    min(exp(sum d), C) ("Diagnosing Training Inference Mismatch in LLM
//    Reinforcement Learning", section 3 on verl's rollout correction;
//    "Rollout-Training Mismatch in LLM RL", section 2.1).
//
// Design: one wave per sequence. Lane l scans the contiguous positions
// [l c, (l+1) c) in order (c = ceil(L / 64)) and folds them into a per-lane
// state; the 64 lane states are then combined in lane order with an XOR
// butterfly whose combine respects the order (lower half on the left), so
// every lane ends with the sequence's result. The order-sensitive fields
// (first mismatch, runs) use a segment monoid; the fp64 sums use the same
// fixed tree, so results are bitwise reproducible and independent of N.
#include <math.h>

#include "lp_internal.h"

namespace lp {
namespace {

struct PairState {
  int first, pre, suf, best;  // order-sensitive (with the shared active count)
  int mism, nonf, k3n;
  double mx, sa, ss, sk, st;
};

struct SeqState {
  int n;  // active tokens in the segment
  PairState p[3];
};

__device__ __forceinline__ void pair_init(PairState& s) {
  s.first = -1;
  s.pre = s.suf = s.best = 0;
  s.mism = s.nonf = s.k3n = 0;
  s.mx = s.sa = s.ss = s.sk = s.st = 0.0;
}

// Fold one active token (active rank k within the segment) into a pair state;
// returns the per-token values |delta|, k3, token TIS (NaN if non-finite).
__device__ __forceinline__ void pair_push(PairState& s, int k, float l, float r,
                                          const CompareArgs& a, float& o_abs,
                                          float& o_k3, float& o_tis) {
  const bool same = __float_as_uint(l) == __float_as_uint(r);
  if (same) {
    // Identical bits: never a mismatch; a finite token adds delta = 0,
    // k3 = 0 and a token TIS weight of min(1, C), so no arithmetic is needed.
    s.suf = 0;
    if (__builtin_isfinite(l)) {
      s.st += fmin(1.0, a.tis_clip);
      o_abs = o_k3 = 0.f;
      o_tis = (float)fmin(1.0, a.tis_clip);
    } else {
      s.nonf += 1;
      o_abs = o_k3 = o_tis = __builtin_nanf("");
    }
    return;
  }
  const double dl = (double)l - (double)r;
  const bool differ = !same && !(a.atol >= 0.0 && fabs(dl) <= a.atol);
  if (differ) {
    if (s.first < 0) s.first = k;
    if (s.pre == k) s.pre = k + 1;  // every token so far differed
    s.suf += 1;
    s.best = max(s.best, s.suf);
    s.mism += 1;
  } else {
    s.suf = 0;
  }
  if (__builtin_isfinite(l) && __builtin_isfinite(r)) {
    const double ad = fabs(dl);
    const double d = -dl;
    double k3, tis;
    if (ad < 0.5) {
      // Small |d| (the common case): fp32 is enough. k3 = expm1(d) - d by
      // its Taylor series (no cancellation; the truncation after d^9/9! is
      // below 2e-9 relative for |d| < 0.5); exp(d) < C needs no clipping
      // unless C < 1.65.
      const float x = (float)d;
      float t = 1.0f / 362880.0f;
      t = __builtin_fmaf(t, x, 1.0f / 40320.0f);
      t = __builtin_fmaf(t, x, 1.0f / 5040.0f);
      t = __builtin_fmaf(t, x, 1.0f / 720.0f);
      t = __builtin_fmaf(t, x, 1.0f / 120.0f);
      t = __builtin_fmaf(t, x, 1.0f / 24.0f);
      t = __builtin_fmaf(t, x, 1.0f / 6.0f);
      t = __builtin_fmaf(t, x, 0.5f);
      k3 = (double)(t * x * x);
      tis = fmin((double)__builtin_amdgcn_exp2f(x * 1.44269504088896341f), a.tis_clip);
    } else {
      k3 = expm1(d) - d;  // fp64: large differences and overflow as defined
      tis = fmin(exp(d), a.tis_clip);
    }
    s.mx = fmax(s.mx, ad);
    s.sa += ad;
    s.ss += dl;
    if (__builtin_isfinite(k3)) s.sk += k3; else s.k3n += 1;
    s.st += tis;
    o_abs = (float)ad;
    o_k3 = (float)k3;
    o_tis = (float)tis;
  } else {
    s.nonf += 1;
    o_abs = o_k3 = o_tis = __builtin_nanf("");
  }
}

// Ordered combine: the segment of L precedes the segment of R.
__device__ __forceinline__ PairState pair_combine(const PairState& L, int nL,
                                                  const PairState& R, int nR) {
  PairState o;
  o.first = L.first >= 0 ? L.first : (R.first >= 0 ? nL + R.first : -1);
  o.pre = (L.pre == nL) ? nL + R.pre : L.pre;
  o.suf = (R.suf == nR) ? nR + L.suf : R.suf;
  o.best = max(max(L.best, R.best), L.suf + R.pre);
  o.mism = L.mism + R.mism;
  o.nonf = L.nonf + R.nonf;
  o.k3n = L.k3n + R.k3n;
  o.mx = fmax(L.mx, R.mx);
  o.sa = L.sa + R.sa;
  o.ss = L.ss + R.ss;
  o.sk = L.sk + R.sk;
  o.st = L.st + R.st;
  return o;
}

__device__ __forceinline__ PairState pair_shfl(const PairState& s, int m) {
  PairState o;
  o.first = __shfl_xor(s.first, m);
  o.pre = __shfl_xor(s.pre, m);
  o.suf = __shfl_xor(s.suf, m);
  o.best = __shfl_xor(s.best, m);
  o.mism = __shfl_xor(s.mism, m);
  o.nonf = __shfl_xor(s.nonf, m);
  o.k3n = __shfl_xor(s.k3n, m);
  o.mx = __shfl_xor(s.mx, m);
  o.sa = __shfl_xor(s.sa, m);
  o.ss = __shfl_xor(s.ss, m);
  o.sk = __shfl_xor(s.sk, m);
  o.st = __shfl_xor(s.st, m);
  return o;
}

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(64 * kWavesPerBlock) void compare_kernel(CompareArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (n >= a.N) return;  // whole wave exits together

  // Lane l scans positions [l c, (l+1) c): c is a multiple of 4 so that the
  // chunk starts are 16-byte aligned; the scalar path visits the same
  // positions in the same order, so both paths give identical bits.
  const int64_t c = (((a.L + 63) / 64) + 3) & ~int64_t(3);
  const int64_t lo = min(a.L, (int64_t)lane * c), hi = min(a.L, lo + c);
  const float* A = a.A + n * a.ld;
  const float* B = a.B + n * a.ld;
  const float* C = a.C + n * a.ld;
  const uint8_t* M = a.mask + n * a.ld;
  const size_t plane = (size_t)a.N * (size_t)a.L;

  SeqState st;
  st.n = 0;
#pragma unroll
  for (int p = 0; p < 3; ++p) pair_init(st.p[p]);

  auto token = [&](int64_t i, float va, float vb, float vc, bool active) {
    float v[3][3] = {{0.f, 0.f, 0.f}, {0.f, 0.f, 0.f}, {0.f, 0.f, 0.f}};
    if (active) {
      const int k = st.n;
      pair_push(st.p[0], k, va, vb, a, v[0][0], v[0][1], v[0][2]);
      pair_push(st.p[1], k, vb, vc, a, v[1][0], v[1][1], v[1][2]);
      pair_push(st.p[2], k, va, vc, a, v[2][0], v[2][1], v[2][2]);
      st.n = k + 1;
    }
    if (a.per_token) {
      float* pt = a.per_token + (size_t)n * a.L + i;
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int q = 0; q < 3; ++q) pt[(size_t)(3 * p + q) * plane] = v[p][q];
    }
  };

  int64_t i = lo;
  if (a.vec) {
    // 16-byte loads of A, B, C and a 4-byte load of the mask per 4 positions,
    // one group of loads kept in flight ahead of the group being folded.
    const int64_t hv = lo + ((hi - lo) & ~int64_t(3));
    if (i < hv) {
      float4 ca = *reinterpret_cast<const float4*>(A + i);
      float4 cb = *reinterpret_cast<const float4*>(B + i);
      float4 cc = *reinterpret_cast<const float4*>(C + i);
      uint32_t cm = *reinterpret_cast<const uint32_t*>(M + i);
      for (; i < hv; i += 4) {
        const int64_t nxt = i + 4 < hv ? i + 4 : i;
        const float4 na = *reinterpret_cast<const float4*>(A + nxt);
        const float4 nb = *reinterpret_cast<const float4*>(B + nxt);
        const float4 nc = *reinterpret_cast<const float4*>(C + nxt);
        const uint32_t nm = *reinterpret_cast<const uint32_t*>(M + nxt);
        token(i + 0, ca.x, cb.x, cc.x, (cm & 0xFFu) != 0);
        token(i + 1, ca.y, cb.y, cc.y, (cm & 0xFF00u) != 0);
        token(i + 2, ca.z, cb.z, cc.z, (cm & 0xFF0000u) != 0);
        token(i + 3, ca.w, cb.w, cc.w, (cm & 0xFF000000u) != 0);
        ca = na; cb = nb; cc = nc; cm = nm;
      }
    }
  }
  for (; i < hi; ++i) token(i, A[i], B[i], C[i], M[i] != 0);

  // Ordered XOR butterfly over the 64 lane segments.
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int on = __shfl_xor(st.n, m);
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const PairState other = pair_shfl(st.p[p], m);
      st.p[p] = upper ? pair_combine(other, on, st.p[p], st.n)
                      : pair_combine(st.p[p], st.n, other, on);
    }
    st.n += on;
  }

  if (lane == 0) {
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      lp_seq_stats* o = a.out + (size_t)p * a.N + n;
      const PairState& s = st.p[p];
      o->valid = st.n;
      o->mismatch = s.mism;
      o->first_div = s.first;
      o->longest_run = s.best;
      o->nonfinite = s.nonf;
      o->k3_nonfinite = s.k3n;
      o->max_abs = s.mx;
      o->sum_abs = s.sa;
      o->sum_signed = s.ss;
      o->sum_k3 = s.sk;
      o->sum_d = -s.ss;  // d = -delta termwise, summed in the same order
      o->seq_tis = fmin(exp(-s.ss), a.tis_clip);
      o->sum_tok_tis = s.st;
    }
  }
}

}  // namespace

hipError_t launch_compare(const CompareArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.N + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(compare_kernel, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace lp
