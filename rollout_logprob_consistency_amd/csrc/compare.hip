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

namespace lp {

// ---------------------------------------------------------------------------
// Batch tail statistics of |delta| per pair (lp_compare_tails): the p50 / p95
// / p99 / max of abs(delta_logprob) that "Diagnosing Training Inference
// Mismatch in LLM Reinforcement Learning" (section 5, practical indicators)
// asks to record, and the logprob_mae / probability_mae numerators with the
// worst token's position of "Fault localization and mismatch bisect" ("Metric
// measurement basis"), plus the error-by-position profile.
//
// Exact order statistics by radix selection on the bit patterns of |delta|
// (non-negative fp64, so the bits order like the values): 8 passes of one
// byte, each a histogram pass over the batch -- one workgroup per sequence,
// LDS counters, integer atomics into 9 global histograms (3 pairs x 3
// quantiles) -- and a one-workgroup select that keeps, per target, the byte
// where the wanted rank falls. Every count is an integer, so the result does
// not depend on the order in which workgroups run. The sums and the first
// worst token are formed per sequence in a fixed order (pass 0) and reduced
// in a fixed tree; the position profile folds fixed chunks of sequences in
// order.
// ---------------------------------------------------------------------------
namespace {

constexpr int kTailTargets = 9;     // 3 pairs x (p50, p95, p99)
constexpr int kTailThreads = 256;
constexpr int kTailChunks = 64;     // sequence chunks of the position profile

struct TailSel {
  uint64_t prefix;   // bytes of the selected key found so far
  int64_t rank;      // 1-based rank still wanted below that prefix; 0: none
};

struct TailPart {    // one (sequence, pair), from pass 0
  double sum_abs, sum_prob;
  uint64_t max_key;  // bits of the largest |delta| (0 without tokens)
  int32_t max_pos;   // its first column, -1 without tokens
  int32_t count;
};

struct TailWs {
  uint32_t* hist;    // [9][256]
  TailSel* sel;      // [9]
  int64_t* count;    // [3]
  TailPart* part;    // [N][3]
  double* pos_part;  // [nch][3][L]
  int32_t* pos_cpart;
  int nch;
};

__host__ __device__ inline size_t tail_up(size_t x) { return (x + 255) & ~size_t(255); }

TailWs tail_layout(void* base, int64_t N, int64_t L) {
  char* p = static_cast<char*>(base);
  TailWs w;
  size_t o = 0;
  w.hist = reinterpret_cast<uint32_t*>(p + o); o = tail_up(o + kTailTargets * 256 * sizeof(uint32_t));
  w.sel = reinterpret_cast<TailSel*>(p + o);   o = tail_up(o + kTailTargets * sizeof(TailSel));
  w.count = reinterpret_cast<int64_t*>(p + o); o = tail_up(o + 3 * sizeof(int64_t));
  w.part = reinterpret_cast<TailPart*>(p + o); o = tail_up(o + (size_t)N * 3 * sizeof(TailPart));
  w.nch = (int)(N < kTailChunks ? (N < 1 ? 1 : N) : kTailChunks);
  w.pos_part = reinterpret_cast<double*>(p + o); o = tail_up(o + (size_t)w.nch * 3 * L * sizeof(double));
  w.pos_cpart = reinterpret_cast<int32_t*>(p + o);
  return w;
}

size_t tail_bytes(int64_t N, int64_t L) {
  size_t o = 0;
  o = tail_up(o + kTailTargets * 256 * sizeof(uint32_t));
  o = tail_up(o + kTailTargets * sizeof(TailSel));
  o = tail_up(o + 3 * sizeof(int64_t));
  o = tail_up(o + (size_t)N * 3 * sizeof(TailPart));
  const int nch = (int)(N < kTailChunks ? (N < 1 ? 1 : N) : kTailChunks);
  o = tail_up(o + (size_t)nch * 3 * L * sizeof(double));
  o = tail_up(o + (size_t)nch * 3 * L * sizeof(int32_t));
  return o;
}

// Left and right side of pair p among the three scores (A, B, C).
__device__ __forceinline__ int pair_left(int p) { return p == 1 ? 1 : 0; }
__device__ __forceinline__ int pair_right(int p) { return p == 0 ? 1 : 2; }

// The target whose histogram target t reads: the first target of its pair
// that is selecting under the same prefix (every one of them in pass 0).
__device__ __forceinline__ int tail_src(const uint64_t* pre, const bool* want, int t) {
  const int p0 = 3 * (t / 3);
  for (int u = p0; u < t; ++u)
    if (want[u] && pre[u] == pre[t]) return u;
  return t;
}

__global__ __launch_bounds__(kTailThreads) void tails_init_kernel(TailWs w) {
  for (int i = threadIdx.x; i < kTailTargets * 256; i += kTailThreads) w.hist[i] = 0u;
  if (threadIdx.x < kTailTargets) w.sel[threadIdx.x] = TailSel{0ull, 0};
}

// One histogram pass; pass 0 also forms the per-sequence sums and maxima.
__global__ __launch_bounds__(kTailThreads) void tails_hist_kernel(TailArgs a, TailWs w, int pass) {
  __shared__ uint32_t h[kTailTargets * 256];
  __shared__ TailPart red[3][kTailThreads];
  const int tid = threadIdx.x;
  for (int i = tid; i < kTailTargets * 256; i += kTailThreads) h[i] = 0u;
  const int shift = 56 - 8 * pass;  // this pass's byte: key bits [shift + 7 : shift]
  // Targets of one pair whose prefixes agree see the same tokens: only the
  // first of them counts (tail_src() below names it for the select kernel).
  uint64_t pre[kTailTargets];
  bool want[kTailTargets];
#pragma unroll
  for (int t = 0; t < kTailTargets; ++t) {
    pre[t] = pass ? w.sel[t].prefix : 0ull;
    want[t] = pass == 0 || w.sel[t].rank > 0;
  }
#pragma unroll
  for (int t = 0; t < kTailTargets; ++t)
    if (tail_src(pre, want, t) != t) want[t] = false;
  __syncthreads();

  const int64_t n = blockIdx.x;
  const float* rows[3] = {a.A + n * a.ld, a.B + n * a.ld, a.C + n * a.ld};
  const uint8_t* M = a.mask + n * a.ld;
  TailPart mine[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) mine[p] = TailPart{0.0, 0.0, 0ull, -1, 0};
  const int lane = tid & 63;
  // Rounded up to whole waves so that every lane of a wave takes part in the
  // ballots below; positions past L are inactive.
  const int64_t Lw = (a.L + kTailThreads - 1) / kTailThreads * kTailThreads;
  for (int64_t i = tid; i < Lw; i += kTailThreads) {
    const bool act = i < a.L && M[i] != 0;
    float v[3] = {0.f, 0.f, 0.f};
    if (act) {
      v[0] = rows[0][i];
      v[1] = rows[1][i];
      v[2] = rows[2][i];
    }
    double e[3] = {0.0, 0.0, 0.0};
    if (pass == 0 && act) {
#pragma unroll
      for (int s = 0; s < 3; ++s)
        if (__builtin_isfinite(v[s])) e[s] = exp_f64((double)v[s]);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const float l = v[pair_left(p)], r = v[pair_right(p)];
      const bool ok = act && __builtin_isfinite(l) && __builtin_isfinite(r);
      const double d = fabs((double)l - (double)r);
      const uint64_t key = (uint64_t)__double_as_longlong(d);
      const uint32_t digit = (uint32_t)(key >> shift) & 255u;
      // After the first passes few tokens share any target's prefix: one
      // ballot per pair lets a wave with no such token skip the targets.
      bool any = ok && pass == 0;
      if (pass != 0) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
          any = any || (ok && want[3 * p + j] && (key >> (shift + 8)) == pre[3 * p + j]);
      }
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int t = 3 * p + j;
        if (!want[t] || __ballot(any) == 0) continue;  // uniform
        const bool hit = ok && (pass == 0 || (key >> (shift + 8)) == pre[t]);
        const uint64_t hb = __ballot(hit);
        if (hb == 0) continue;
        // One atomic for the wave when all its hits share a bin (the common
        // case: runs of identical scores put every lane in bin 0).
        const int first = __ffsll((long long)hb) - 1;
        const uint32_t d0 = (uint32_t)__shfl((int)digit, first);
        if (__ballot(hit && digit != d0) == 0) {
          if (lane == first) atomicAdd(&h[t * 256 + d0], (uint32_t)__popcll(hb));
        } else if (hit) {
          atomicAdd(&h[t * 256 + digit], 1u);
        }
      }
      if (!ok) continue;
      if (pass == 0) {
        TailPart& m = mine[p];
        m.sum_abs += d;
        m.sum_prob += fabs(e[pair_left(p)] - e[pair_right(p)]);
        if (m.max_pos < 0 || key > m.max_key) {  // positions ascend: the first one stays
          m.max_key = key;
          m.max_pos = (int32_t)i;
        }
        m.count += 1;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < kTailTargets * 256; i += kTailThreads)
    if (h[i]) atomicAdd(&w.hist[i], h[i]);
  if (pass != 0) return;

  // Fixed tree over the threads (thread t holds the columns = t mod 256).
#pragma unroll
  for (int p = 0; p < 3; ++p) red[p][tid] = mine[p];
  __syncthreads();
  for (int stride = kTailThreads / 2; stride > 0; stride >>= 1) {
    if (tid < stride) {
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        TailPart x = red[p][tid];
        const TailPart y = red[p][tid + stride];
        x.sum_abs += y.sum_abs;
        x.sum_prob += y.sum_prob;
        x.count += y.count;
        if (y.max_pos >= 0 &&
            (x.max_pos < 0 || y.max_key > x.max_key || (y.max_key == x.max_key && y.max_pos < x.max_pos))) {
          x.max_key = y.max_key;
          x.max_pos = y.max_pos;
        }
        red[p][tid] = x;
      }
    }
    __syncthreads();
  }
  if (tid < 3) w.part[n * 3 + tid] = red[tid][0];
}

// Select the byte of each target's key; one wave per target, 4 bins a lane.
// A target reads the histogram of tail_src() (the same prefix within its
// pair); every histogram is read before any is cleared or any prefix moves.
__global__ __launch_bounds__(64 * kTailTargets) void tails_select_kernel(TailWs w, int pass) {
  const int t = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t pre[kTailTargets];
  bool want[kTailTargets];
#pragma unroll
  for (int u = 0; u < kTailTargets; ++u) {
    pre[u] = pass ? w.sel[u].prefix : 0ull;
    want[u] = pass == 0 || w.sel[u].rank > 0;
  }
  const int src = tail_src(pre, want, t);
  const uint32_t* hist = w.hist + src * 256;
  uint32_t c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) c[k] = hist[4 * lane + k];
  const int64_t old_rank = pass ? w.sel[t].rank : 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) w.hist[t * 256 + 4 * lane + k] = 0u;
  const int64_t lsum = (int64_t)c[0] + c[1] + c[2] + c[3];
  int64_t incl = lsum;  // inclusive scan over lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const int64_t total = __shfl(incl, 63);
  int64_t rank;
  if (pass == 0) {
    // The pass-0 histogram holds every counted token of the pair.
    const int64_t pct = (t % 3 == 0) ? 50 : (t % 3 == 1 ? 95 : 99);
    rank = total > 0 ? (pct * total + 99) / 100 : 0;
    if (t % 3 == 0 && lane == 0) w.count[t / 3] = total;
  } else {
    rank = old_rank;
  }
  const int64_t excl = incl - lsum;
  if (rank > 0 && excl < rank && rank <= incl) {
    int64_t below = excl;
    int k = 0;
    while (below + (int64_t)c[k] < rank) below += c[k++];
    w.sel[t].prefix = (pass ? (pre[t] << 8) : 0ull) | (uint64_t)(4 * lane + k);
    w.sel[t].rank = rank - below;
  } else if (rank == 0 && lane == 0) {
    w.sel[t].rank = 0;
  }
}

// Batch results per pair: fixed chunks of sequences per thread, fixed tree.
__global__ __launch_bounds__(kTailThreads) void tails_final_kernel(TailArgs a, TailWs w) {
  __shared__ TailPart red[kTailThreads];
  __shared__ int32_t red_seq[kTailThreads];
  const int tid = threadIdx.x;
  const int64_t per = (a.N + kTailThreads - 1) / kTailThreads;
  for (int p = 0; p < 3; ++p) {
    TailPart x{0.0, 0.0, 0ull, -1, 0};
    int32_t xs = -1;
    const int64_t lo = tid * per, hi = min(a.N, lo + per);
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
    red[tid] = x;
    red_seq[tid] = xs;
    __syncthreads();
    for (int stride = kTailThreads / 2; stride > 0; stride >>= 1) {
      if (tid < stride) {
        TailPart u = red[tid];
        const TailPart v = red[tid + stride];
        u.sum_abs += v.sum_abs;
        u.sum_prob += v.sum_prob;
        u.count += v.count;
        // After the first steps a thread's sequences interleave with its
        // partner's, so an equal key is decided by the sequence index.
        const int32_t us = red_seq[tid], vs = red_seq[tid + stride];
        if (v.max_pos >= 0 &&
            (u.max_pos < 0 || v.max_key > u.max_key || (v.max_key == u.max_key && vs < us))) {
          u.max_key = v.max_key;
          u.max_pos = v.max_pos;
          red_seq[tid] = vs;
        }
        red[tid] = u;
      }
      __syncthreads();
    }
    if (tid == 0) {
      const TailPart& r = red[0];
      lp_tail_stats o;
      o.count = w.count[p];
      const bool any = o.count > 0;
      o.q50 = any ? __longlong_as_double((long long)w.sel[3 * p].prefix) : 0.0;
      o.q95 = any ? __longlong_as_double((long long)w.sel[3 * p + 1].prefix) : 0.0;
      o.q99 = any ? __longlong_as_double((long long)w.sel[3 * p + 2].prefix) : 0.0;
      o.max_abs = any ? __longlong_as_double((long long)r.max_key) : 0.0;
      o.max_seq = any ? red_seq[0] : -1;
      o.max_pos = any ? r.max_pos : -1;
      o.sum_abs = r.sum_abs;
      o.sum_prob_abs = r.sum_prob;
      a.out[p] = o;
    }
    __syncthreads();
  }
}

// Position profile, stage 1: chunk c of the sequences, column i.
__global__ __launch_bounds__(kTailThreads) void tails_pos_kernel(TailArgs a, TailWs w) {
  const int64_t i = (int64_t)blockIdx.x * kTailThreads + threadIdx.x;
  if (i >= a.L) return;
  const int c = blockIdx.y;
  const int64_t per = (a.N + w.nch - 1) / w.nch;
  const int64_t lo = c * per, hi = min(a.N, lo + per);
  double s[3] = {0.0, 0.0, 0.0};
  int32_t k[3] = {0, 0, 0};
  for (int64_t n = lo; n < hi; ++n) {
    const int64_t o = n * a.ld + i;
    if (a.mask[o] == 0) continue;
    const float v[3] = {a.A[o], a.B[o], a.C[o]};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const float l = v[pair_left(p)], r = v[pair_right(p)];
      if (!__builtin_isfinite(l) || !__builtin_isfinite(r)) continue;
      s[p] += fabs((double)l - (double)r);
      k[p] += 1;
    }
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    w.pos_part[((size_t)c * 3 + p) * a.L + i] = s[p];
    w.pos_cpart[((size_t)c * 3 + p) * a.L + i] = k[p];
  }
}

// Position profile, stage 2: fold the chunks in order.
__global__ __launch_bounds__(kTailThreads) void tails_pos_fold_kernel(TailArgs a, TailWs w) {
  const int64_t idx = (int64_t)blockIdx.x * kTailThreads + threadIdx.x;  // p * L + i
  if (idx >= 3 * a.L) return;
  double s = 0.0;
  int32_t k = 0;
  for (int c = 0; c < w.nch; ++c) {
    s += w.pos_part[(size_t)c * 3 * a.L + idx];
    k += w.pos_cpart[(size_t)c * 3 * a.L + idx];
  }
  a.pos_sum[idx] = s;
  a.pos_count[idx] = k;
}

}  // namespace

size_t tails_workspace_bytes(int64_t N, int64_t L) { return tail_bytes(N, L); }

hipError_t launch_tails(const TailArgs& a, hipStream_t stream) {
  const TailWs w = tail_layout(a.workspace, a.N, a.L);
  hipLaunchKernelGGL(tails_init_kernel, dim3(1), dim3(kTailThreads), 0, stream, w);
  if (a.N > 0) {
    // Every pass runs, also with L == 0 (pass 0 then writes empty partials).
    for (int pass = 0; pass < 8; ++pass) {
      hipLaunchKernelGGL(tails_hist_kernel, dim3((unsigned)a.N), dim3(kTailThreads), 0, stream,
                         a, w, pass);
      hipLaunchKernelGGL(tails_select_kernel, dim3(1), dim3(64 * kTailTargets), 0, stream, w,
                         pass);
    }
  } else {
    // No sequence: empty histograms give count 0 and no rank to select.
    hipLaunchKernelGGL(tails_select_kernel, dim3(1), dim3(64 * kTailTargets), 0, stream, w, 0);
  }
  hipLaunchKernelGGL(tails_final_kernel, dim3(1), dim3(kTailThreads), 0, stream, a, w);
  if (a.pos_sum && a.L > 0) {
    // Stage 1 also runs with N == 0, writing zero partials for the fold.
    hipLaunchKernelGGL(tails_pos_kernel,
                       dim3((unsigned)((a.L + kTailThreads - 1) / kTailThreads), (unsigned)w.nch),
                       dim3(kTailThreads), 0, stream, a, w);
    hipLaunchKernelGGL(tails_pos_fold_kernel,
                       dim3((unsigned)((3 * a.L + kTailThreads - 1) / kTailThreads)),
                       dim3(kTailThreads), 0, stream, a, w);
  }
  return hipGetLastError();
}

}  // namespace lp
