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
//    that in fp64 from one exponential, (e^d - 1) - d;
//  * token and sequence truncated importance weights min(exp(d), C) and
//    min(exp(sum d), C) ("Diagnosing Training Inference Mismatch in LLM
//    Reinforcement Learning", section 3 on verl's rollout correction;
//    "Rollout-Training Mismatch in LLM RL", section 2.1).
//
// Design: one workgroup per sequence, one wave per pair, so each wave keeps
// the state of a single pair (few registers, high occupancy). A wave walks its
// sequence in windows of 256 positions; lane l folds positions w + 4l ..
// w + 4l + 3 (one 16-byte load per score array and a 4-byte mask load, so
// every load instruction reads one contiguous KiB), with the next window's
// loads in flight. Statistics that do not depend on order -- counts, max and
// the fp64 sums -- accumulate per lane across windows. The order-sensitive
// ones (first mismatch and runs, a segment monoid over the active tokens) are
// formed per window -- from ballots when the window is all-equal or
// all-different, else by an ordered XOR butterfly whose lower half is always
// the left operand -- and folded into the sequence state in window order. The
// per-lane accumulators are reduced at the end by a fixed XOR butterfly (each
// step adds the same two values in both lanes). Everything depends only on L,
// so results are bitwise reproducible and independent of N. The three waves
// read the mask and each score array twice; the second reads hit in cache.
#include <math.h>

#include "lp_internal.h"

namespace lp {
namespace {

constexpr int kWindow = 256;  // positions per wave step (64 lanes x 4)

// Order-sensitive state of one pair over a segment of active tokens.
struct Runs {
  int first, pre, suf, best;
};

// Ordered combine: the segment of L (nL active tokens) precedes that of R.
__device__ __forceinline__ Runs runs_combine(const Runs& L, int nL, const Runs& R, int nR) {
  Runs o;
  o.first = L.first >= 0 ? L.first : (R.first >= 0 ? nL + R.first : -1);
  o.pre = (L.pre == nL) ? nL + R.pre : L.pre;
  o.suf = (R.suf == nR) ? nR + L.suf : R.suf;
  o.best = max(max(L.best, R.best), L.suf + R.pre);
  return o;
}

// e^x in fp64 for finite x (the rare tokens with |d| >= 0.5). Cody-Waite
// reduction x = k ln2 + r with ln2 split into a 32-bit head (k * head is exact
// for |k| < 2^21) and a tail, |r| <= ln2 / 2; e^r by its Taylor series to
// degree 12 (truncation < 2e-16 relative); then the exact scaling by 2^k,
// which overflows to +inf and underflows to 0 as the true value does. x is
// clamped to [-800, 800] first, beyond which e^x is already inf or 0.
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

// 7 waves per SIMD: the 68 registers this allows hold the whole state without
// spilling (at 8 waves the spill area of 24 bytes per lane cost more write
// traffic than the extra wave saved).
__global__ __launch_bounds__(192) __attribute__((amdgpu_waves_per_eu(7))) void compare_kernel(
    CompareArgs a) {
  const int lane = threadIdx.x & 63;
  const int p = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // pair of this wave
  const int64_t n = blockIdx.x;
  const float* Lp = (p == 1 ? a.B : a.A) + n * a.ld;
  const float* Rp = (p == 0 ? a.B : a.C) + n * a.ld;
  const uint8_t* M = a.mask + n * a.ld;
  const size_t plane = (size_t)a.N * (size_t)a.L;
  float* pt_row = a.per_token ? a.per_token + (size_t)(3 * p) * plane + (size_t)n * a.L : nullptr;
  const double clip = a.tis_clip;
  const double one_tis = fmin(1.0, clip);  // TIS weight of a token with d = 0
  const float nan = __builtin_nanf("");

  int seq_n = 0;  // active tokens folded so far (same in every lane)
  Runs seq = {-1, 0, 0, 0};
  int mism = 0, nonf = 0, k3n = 0;
  double mx = 0.0, sa = 0.0, ss = 0.0, sk = 0.0, st = 0.0;
  bool slow = false;  // this lane has a finite token with |d| >= 0.5

  // Folds the window holding positions i0 .. i0 + 3 of this lane.
  auto fold = [&](int64_t i0, const float (&vl)[4], const float (&vr)[4], unsigned amask) {
      unsigned dif = 0, bad = 0;  // bit e: mismatch / non-finite
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float o_abs = 0.f, o_k3 = 0.f, o_tis = 0.f;
        if ((amask >> e) & 1u) {
          const float l = vl[e], r = vr[e];
          if (__float_as_uint(l) == __float_as_uint(r)) {
            // Identical bits: never a mismatch; a finite token adds delta = 0,
            // k3 = 0 and a TIS weight of min(1, C), so no arithmetic is needed.
            if (__builtin_isfinite(l)) {
              st += one_tis;
              o_tis = (float)one_tis;
            } else {
              bad |= 1u << e;
              o_abs = o_k3 = o_tis = nan;
            }
          } else {
            const double dl = (double)l - (double)r;  // non-finite iff l or r is
            const double ad = fabs(dl);
            // atol < 0 (bitwise mode) never holds here, nor does a NaN delta.
            if (!(ad <= a.atol)) dif |= 1u << e;
            if (__builtin_isfinite(dl)) {
              mx = ad > mx ? ad : mx;
              sa += ad;
              ss += dl;
              o_abs = (float)ad;
              if (ad < 0.5) {
                // fp32 is enough: k3 = expm1(d) - d by its Taylor series (no
                // cancellation; truncation after d^9/9! < 2e-9 relative).
                const float x = (float)-dl;
                float t = 1.0f / 362880.0f;
                t = __builtin_fmaf(t, x, 1.0f / 40320.0f);
                t = __builtin_fmaf(t, x, 1.0f / 5040.0f);
                t = __builtin_fmaf(t, x, 1.0f / 720.0f);
                t = __builtin_fmaf(t, x, 1.0f / 120.0f);
                t = __builtin_fmaf(t, x, 1.0f / 24.0f);
                t = __builtin_fmaf(t, x, 1.0f / 6.0f);
                t = __builtin_fmaf(t, x, 0.5f);
                const float k3 = t * x * x;
                const double tis =
                    fmin((double)__builtin_amdgcn_exp2f(x * 1.44269504088896341f), clip);
                sk += (double)k3;
                st += tis;
                o_k3 = k3;
                o_tis = (float)tis;
              } else {
                slow = true;  // k3 and TIS in the second pass
              }
            } else {
              bad |= 1u << e;
              o_abs = o_k3 = o_tis = nan;
            }
          }
        }
        if (pt_row && i0 + e < a.L) {
          pt_row[i0 + e] = o_abs;
          pt_row[plane + i0 + e] = o_k3;
          pt_row[2 * plane + i0 + e] = o_tis;
        }
      }
      mism += __popc(dif);
      nonf += __popc(bad);

      int wn = 0;  // active tokens in this window
#pragma unroll
      for (int e = 0; e < 4; ++e) wn += __popcll(__ballot((amask >> e) & 1u));
      Runs win;
      if (__ballot(dif != 0u) == 0) {
        win = {-1, 0, 0, 0};  // no mismatch
      } else if (__ballot((amask & ~dif) != 0u) == 0) {
        win = {0, wn, wn, wn};  // every active token mismatches
      } else {
        Runs s = {-1, 0, 0, 0};
        int k = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((amask >> e) & 1u) {
            if ((dif >> e) & 1u) {
              if (s.first < 0) s.first = k;
              if (s.pre == k) s.pre = k + 1;  // every token so far differed
              s.suf += 1;
              s.best = max(s.best, s.suf);
            } else {
              s.suf = 0;
            }
            ++k;
          }
        }
        int sn = k;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          Runs o;
          o.first = __shfl_xor(s.first, m);
          o.pre = __shfl_xor(s.pre, m);
          o.suf = __shfl_xor(s.suf, m);
          o.best = __shfl_xor(s.best, m);
          const int on = __shfl_xor(sn, m);
          s = (lane & m) ? runs_combine(o, on, s, sn) : runs_combine(s, sn, o, on);
          sn += on;
        }
        win = s;
      }
      seq = runs_combine(seq, seq_n, win, wn);
      seq_n += wn;
  };

  // Windows that lie wholly inside the row take 16-byte loads (when the rows
  // allow them), with the next window's loads issued before the current one
  // is folded; the last load repeats a window instead of branching. The
  // remaining partial window, and every window of unaligned rows, takes
  // element loads. Both visit the same positions in the same order.
  const int64_t full = a.vec ? (a.L / kWindow) * kWindow : 0;
  const int64_t l4 = 4 * lane;
  if (full > 0) {
    float4 ql = *reinterpret_cast<const float4*>(Lp + l4);
    float4 qr = *reinterpret_cast<const float4*>(Rp + l4);
    uint32_t qm = *reinterpret_cast<const uint32_t*>(M + l4);
    for (int64_t w = 0; w < full; w += kWindow) {
      const int64_t nx = min(w + kWindow, full - kWindow) + l4;
      const float4 nl = *reinterpret_cast<const float4*>(Lp + nx);
      const float4 nr = *reinterpret_cast<const float4*>(Rp + nx);
      const uint32_t nm = *reinterpret_cast<const uint32_t*>(M + nx);
      const float vl[4] = {ql.x, ql.y, ql.z, ql.w};
      const float vr[4] = {qr.x, qr.y, qr.z, qr.w};
      unsigned amask = 0;  // bit e: position w + l4 + e is active
#pragma unroll
      for (int e = 0; e < 4; ++e) amask |= (((qm >> (8 * e)) & 0xFFu) != 0 ? 1u : 0u) << e;
      fold(w + l4, vl, vr, amask);
      ql = nl;
      qr = nr;
      qm = nm;
    }
  }
  for (int64_t w = full; w < a.L; w += kWindow) {
    const int64_t i0 = w + l4;
    float vl[4], vr[4];
    unsigned amask = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool act = i0 + e < a.L && M[i0 + e] != 0;
      amask |= (act ? 1u : 0u) << e;
      vl[e] = act ? Lp[i0 + e] : 0.f;
      vr[e] = act ? Rp[i0 + e] : 0.f;
    }
    fold(i0, vl, vr, amask);
  }

  // Second pass, only for rows that have tokens with |d| >= 0.5: their k3 and
  // TIS terms in fp64 from one exponential, (e^d - 1) - d (no cancellation at
  // that size). Same positions per lane; the terms are summed apart and added
  // once, so the order stays a fixed function of the row.
  if (__ballot(slow) != 0) {
    double sk2 = 0.0, st2 = 0.0;
    for (int64_t w = 0; w < a.L; w += kWindow) {
#pragma unroll 1
      for (int e = 0; e < 4; ++e) {
        const int64_t i = w + 4 * lane + e;
        if (i >= a.L || M[i] == 0) continue;
        const double dl = (double)Lp[i] - (double)Rp[i];
        if (!(fabs(dl) >= 0.5) || !__builtin_isfinite(dl)) continue;
        const double d = -dl;
        const double E = exp_f64(d);
        const double k3 = (E - 1.0) - d;
        const double tis = fmin(E, clip);
        if (__builtin_isfinite(k3)) sk2 += k3; else k3n += 1;
        st2 += tis;
        if (pt_row) {
          pt_row[plane + i] = (float)k3;
          pt_row[2 * plane + i] = (float)tis;
        }
      }
    }
    sk += sk2;
    st += st2;
  }

#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    mism += __shfl_xor(mism, m);
    nonf += __shfl_xor(nonf, m);
    k3n += __shfl_xor(k3n, m);
    const double omx = __shfl_xor(mx, m);
    mx = omx > mx ? omx : mx;
    sa += __shfl_xor(sa, m);
    ss += __shfl_xor(ss, m);
    sk += __shfl_xor(sk, m);
    st += __shfl_xor(st, m);
  }

  if (lane == 0) {
    lp_seq_stats* o = a.out + (size_t)p * a.N + n;
    o->valid = seq_n;
    o->mismatch = mism;
    o->first_div = seq.first;
    o->longest_run = seq.best;
    o->nonfinite = nonf;
    o->k3_nonfinite = k3n;
    o->max_abs = mx;
    o->sum_abs = sa;
    o->sum_signed = ss;
    o->sum_k3 = sk;
    o->sum_d = -ss;  // d = -delta termwise, summed in the same order
    o->seq_tis = fmin(exp(-ss), clip);
    o->sum_tok_tis = st;
  }
}

}  // namespace

hipError_t launch_compare(const CompareArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(compare_kernel, dim3((unsigned)a.N), dim3(192), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lp
