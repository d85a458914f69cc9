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
//    exponential terms are evaluated in fp32 (k3 by a fitted polynomial of
//    its series), beyond that in fp64 from one exponential, (e^d - 1) - d;
//  * token and sequence truncated importance weights min(exp(d), C) and
//    min(exp(sum d), C) ("Diagnosing Training Inference Mismatch in LLM
//    Reinforcement Learning", section 3 on verl's rollout correction;
//    "Rollout-Training Mismatch in LLM RL", section 2.1).
//
// Design: one workgroup per sequence, one wave per pair, so each wave keeps
// the state of a single pair (few registers, high occupancy). The sequence is
// walked in windows of 256 positions; lane l folds positions w + 4l ..
// w + 4l + 3. Each wave copies one of the three score arrays (and the mask)
// of a window from memory straight into a four-window LDS ring (buffer ->
// LDS loads, every array read once, three windows in flight, no VGPR held by
// a load), and the pair waves read their two arrays from the ring. Most
// windows are empty (prompt, padding), all-mismatching with small
// differences, or all-identical, and take wave-uniform shortcuts; the others
// take the general fold. Statistics that do not depend on order -- counts,
// max and the fp64 sums -- accumulate per lane across windows. The
// order-sensitive ones (first mismatch and runs, a segment monoid over the
// active tokens) are formed per window -- from ballots when the window's
// active tokens all agree or all differ, else by an ordered XOR butterfly
// whose lower half is always the left operand -- and folded into the
// sequence state in window order. The per-lane accumulators are reduced at
// the end by a fixed XOR butterfly (each step adds the same two values in
// both lanes). Everything depends only on L, so results are bitwise
// reproducible and independent of N.
#include <math.h>

#include <type_traits>

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

// k3 and e^x of a token with |x| < 0.5 in fp32: k3 = expm1(x) - x =
// x^2 g(x) with g(x) = sum_k x^k / (k + 2)! (no cancellation), g by a
// degree-5 polynomial fitted on [-0.5, 0.5] (Chebyshev nodes, then least
// squares reweighted toward equal relative error): 2.5e-8 relative in exact
// arithmetic, below fp32 rounding. Returns t x (so k3 = (t x) x, which the
// caller folds into its sum with one fma) and e^x - 1 = x + k3, formed from
// the same series with no exponential instruction (rounding about 1e-7
// relative). Every path of the kernel goes through this one function, so a
// token's terms have the same bits whichever path folds it.
__device__ __forceinline__ float small_tx(float x) {
  float t = 1.9875631549451514e-4f;
  t = __builtin_fmaf(t, x, 1.3982032161686808e-3f);
  t = __builtin_fmaf(t, x, 8.333452311488566e-3f);
  t = __builtin_fmaf(t, x, 4.166579533613375e-2f);
  t = __builtin_fmaf(t, x, 1.666666545420338e-1f);
  t = __builtin_fmaf(t, x, 5.000000120251578e-1f);
  return t * x;
}

// min(e^x, C) of a small-|x| token from t x: 1 + (x + k3), capped by one
// v_min (both operands finite; fminf would first canonicalize them).
__device__ __forceinline__ float small_tis(float tx, float x, float clip_f) {
  float tis;
  asm("v_min_f32 %0, %1, %2" : "=v"(tis) : "v"(1.0f + __builtin_fmaf(tx, x, x)), "v"(clip_f));
  return tis;
}

// ---- Window ring: the score arrays of a sequence go from memory straight
// into LDS (buffer_load ... lds: no VGPR holds a load in flight), each array
// once per workgroup, and the three pair waves read their two arrays from
// there. kRing windows are in the ring; kRing - 1 are in flight.
typedef __attribute__((address_space(3))) char lds_char;
constexpr int kRing = 4;
constexpr int kSlotB = 3 * 1024 + 3 * 256;  // A, B, C (256 fp32 each), one mask copy per wave

// One buffer -> LDS copy: lane i moves 16 bytes (kDw4) or 4 bytes from
// rsrc + voff + soff to LDS byte lds + 16 i (or 4 i). Inline assembly, so the
// compiler does not take the asynchronous LDS write as aliasing every LDS
// read that follows (it would wait for all copies in flight); the ring's
// vmcnt waits and barriers order copies and reads. M0 holds the LDS address.
// The compiler inserts no wait states before an inline-assembly instruction,
// so the statement carries its own: 5, which covers both an M0 write (1) and
// a VALU write of the resource or offset SGPRs (5; e.g. a v_readlane that
// restores a spilled resource), and the build checks the result.
template <bool kDw4>
__device__ __forceinline__ void ring_copy(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, uint32_t voff,
                                          uint32_t soff) {
  if (kDw4)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
                 : "memory");
  else
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
                 : "memory");
}

// Instantiated for per-token output requested or not (kPT) and for the
// bitwise mismatch test or the atol one (kBitwise), so the common call
// carries no per-token bookkeeping and no tolerance test.
template <bool kPT, bool kBitwise, bool kTisCount>
__global__ __launch_bounds__(192) __attribute__((amdgpu_waves_per_eu(8))) void compare_kernel(
    CompareArgs a) {
  __shared__ __attribute__((aligned(1024))) char ring[kRing * kSlotB];
  const int lane = threadIdx.x & 63;
  const int p = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // pair of this wave
  // Workgroups are dealt to the 8 XCDs in turn; XCD x takes the x-th
  // contiguous eighth of the sequences, so that the records of neighbouring
  // sequences (and their rows) meet in one L2 and leave it as whole lines
  // rather than as partial lines from several XCDs.
  int64_t n;
  {
    const int64_t b = blockIdx.x, xcd = b & 7, idx = b >> 3, per = a.N >> 3, rem = a.N & 7;
    n = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  }
  const float* Lp = (p == 1 ? a.B : a.A) + n * a.ld;
  const float* Rp = (p == 0 ? a.B : a.C) + n * a.ld;
  const uint8_t* M = a.mask + n * a.ld;
  const size_t plane = (size_t)a.N * (size_t)a.L;
  float* pt_row = kPT ? a.per_token + (size_t)(3 * p) * plane + (size_t)n * a.L : nullptr;
  const double clip = a.tis_clip;
  const float clip_f = (float)clip;  // exact: the cap is given in fp32
  const float one_tis = fminf(1.0f, clip_f);  // TIS weight of a token with d = 0
  // With C > e^0.5 (kTisCount) no token with |d| < 0.5 reaches the cap, so
  // the sum of their weights e^d = 1 + d + k3 is formed from the count of
  // such tokens, their sum of d and their sum of k3 (all kept anyway); only
  // the tokens with |d| >= 0.5 take min(e^d, C) one by one. Below that cap
  // each token's weight is capped and summed.
  constexpr bool tis_count = kTisCount;  // the cap is above e^0.5 (the launch checks)
  const float nan = __builtin_nanf("");

  int seq_n = 0;  // active tokens folded so far (same in every lane)
  Runs seq = {-1, 0, 0, 0};
  int mism = 0, nonf = 0, k3n = 0;
  int mism_w = 0;  // mismatches counted a whole window at a time (wave-uniform)
  double mx = 0.0, sa = 0.0, ss = 0.0, sk = 0.0, st = 0.0;
  bool slow = false;  // this lane has a finite token with |d| >= 0.5

  // Folds the window holding positions i0 .. i0 + 3 of this lane.
  auto fold = [&](int64_t i0, const float (&vl)[4], const float (&vr)[4], unsigned amask) {
      unsigned dif = 0, bad = 0;  // bit e: mismatch / non-finite
      // The window's k3 and TIS terms (all >= 0) are summed in fp32 and
      // added to the fp64 sums once: at most 3 roundings of 2^-24 relative.
      float wk = 0.f, wt = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float o_abs = 0.f, o_k3 = 0.f, o_tis = 0.f;
        if ((amask >> e) & 1u) {
          const float l = vl[e], r = vr[e];
          if (__float_as_uint(l) == __float_as_uint(r)) {
            // Identical bits: never a mismatch; a finite token adds delta = 0,
            // k3 = 0 and a TIS weight of min(1, C), so no arithmetic is needed.
            if (__builtin_isfinite(l)) {
              wt += one_tis;
              o_tis = one_tis;
            } else {
              bad |= 1u << e;
              o_abs = o_k3 = o_tis = nan;
            }
          } else {
            const double dl = (double)l - (double)r;  // non-finite iff l or r is
            const double ad = fabs(dl);
            // Different bits are a mismatch; with atol, unless |delta| <= atol
            // (never true for a NaN delta).
            if (kBitwise || !(ad <= a.atol)) dif |= 1u << e;
            if (__builtin_isfinite(dl)) {
              // Both finite and >= 0: one v_max is the exact maximum (fmax
              // would first canonicalize both operands).
              asm("v_max_f64 %0, |%1|, %2" : "=v"(mx) : "v"(dl), "v"(mx));
              sa += ad;
              ss += dl;
              o_abs = (float)ad;
              if (ad < 0.5) {
                const float x = r - l;  // d in fp32 (within an ulp of -dl)
                const float tx = small_tx(x);
                wk = __builtin_fmaf(tx, x, wk);
                if (kPT || !tis_count) {
                  const float tis = small_tis(tx, x, clip_f);
                  wt += tis;
                  o_k3 = tx * x;
                  o_tis = tis;
                }
              } else {
                slow = true;  // k3 and TIS in the second pass
              }
            } else {
              bad |= 1u << e;
              o_abs = o_k3 = o_tis = nan;
            }
          }
        }
        if (kPT && i0 + e < a.L) {
          pt_row[i0 + e] = o_abs;
          pt_row[plane + i0 + e] = o_k3;
          pt_row[2 * plane + i0 + e] = o_tis;
        }
      }
      sk += (double)wk;
      if (!tis_count) st += (double)wt;
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
        // Ordered XOR butterfly: the lower lanes' segment is the left operand.
        auto step = [&](auto m_tag, int m) __attribute__((always_inline)) {
          constexpr int kM = decltype(m_tag)::value;
          Runs o;
          o.first = xlane<kM>(s.first);
          o.pre = xlane<kM>(s.pre);
          o.suf = xlane<kM>(s.suf);
          o.best = xlane<kM>(s.best);
          const int on = xlane<kM>(sn);
          s = (lane & m) ? runs_combine(o, on, s, sn) : runs_combine(s, sn, o, on);
          sn += on;
        };
        step(std::integral_constant<int, 1>{}, 1);
        step(std::integral_constant<int, 2>{}, 2);
        step(std::integral_constant<int, 4>{}, 4);
        step(std::integral_constant<int, 8>{}, 8);
        step(std::integral_constant<int, 16>{}, 16);
        // Step 32: each 32-lane half is uniform; lanes 0 and 32 hold them.
        const Runs lo = {lane_value(s.first, 0), lane_value(s.pre, 0), lane_value(s.suf, 0),
                         lane_value(s.best, 0)};
        const Runs hi = {lane_value(s.first, 32), lane_value(s.pre, 32), lane_value(s.suf, 32),
                         lane_value(s.best, 32)};
        win = runs_combine(lo, lane_value(sn, 0), hi, lane_value(sn, 32));
      }
      seq = runs_combine(seq, seq_n, win, wn);
      seq_n += wn;
  };

  // Windows that lie wholly inside the row go through the LDS ring (when the
  // rows are 16-byte aligned and at most 2^28 positions long, so that buffer
  // offsets fit in 32 bits). The remaining partial window, and every window
  // of other rows, takes element loads. Both visit the same positions in the
  // same order and fold them the same way.
  const int64_t full = (a.vec && a.L <= (int64_t(1) << 28)) ? (a.L / kWindow) * kWindow : 0;
  const int64_t l4 = 4 * lane;
  if (full > 0) {
    // Window k sits in ring slot k mod kRing. Wave p copies array p (A, B or
    // C: 256 values, one 16-byte chunk a lane) and its own copy of the mask
    // bytes; a copy index past the last window repeats the last window, so
    // every wave issues two copies per window and the counts stay exact.
    const int nwin = (int)(full / kWindow);
    const float* Xp = (p == 0 ? a.A : (p == 1 ? a.B : a.C)) + n * a.ld;
    const __amdgpu_buffer_rsrc_t xres = row_rsrc(Xp, (uint32_t)(full * 4));
    const __amdgpu_buffer_rsrc_t mres = row_rsrc(M, (uint32_t)full);
    const uint32_t ring0 =
        __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_char*)ring));
    auto issue = [&](int k) __attribute__((always_inline)) {
      const int kc = min(k, nwin - 1);
      const uint32_t slot = ring0 + (uint32_t)(k % kRing) * kSlotB;
      ring_copy<true>(xres, slot + 1024u * (uint32_t)p, 16u * (uint32_t)lane, (uint32_t)kc * 1024u);
      ring_copy<false>(mres, slot + 3072u + 256u * (uint32_t)p, 4u * (uint32_t)lane,
                       (uint32_t)kc * 256u);
    };
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k) issue(k);
    const int lo = p == 1 ? 1 : 0, ro = p == 0 ? 1 : 2;  // arrays of this pair
    for (int k = 0; k < nwin; ++k) {
      const int64_t w = (int64_t)k * kWindow;
      // This wave's copies of window k have landed once at most the
      // 2 (kRing - 2) younger ones are outstanding (vector memory counts
      // retire in issue order; with per-token stores in the loop, wait for
      // all). After the barrier every wave's copies of window k are in LDS
      // and every wave has finished reading window k - 1, whose slot takes
      // window k + kRing - 1.
      if (kPT) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      else __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * (kRing - 2)));
      __syncthreads();
      issue(k + kRing - 1);
      const char* slot = ring + (k % kRing) * kSlotB;
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      f32x4 ql = *reinterpret_cast<const f32x4*>(slot + 1024 * lo + 16 * lane);
      f32x4 qr = *reinterpret_cast<const f32x4*>(slot + 1024 * ro + 16 * lane);
      uint32_t qm = *reinterpret_cast<const uint32_t*>(slot + 3072 + 256 * p + 4 * lane);
      // The three reads go out together (one LDS round trip, not the mask's
      // and then the scores' after the empty-window test).
      asm volatile("" : "+v"(ql), "+v"(qr), "+v"(qm));
      const float vl[4] = {ql[0], ql[1], ql[2], ql[3]};
      const float vr[4] = {qr[0], qr[1], qr[2], qr[3]};
      // Three wave-uniform shortcuts for the common windows; the folds they
      // make are exactly the general fold's for those windows, term by term
      // and in the same order. Conditions are gathered as wave masks (one
      // compare each, combined in scalar registers); all 64 lanes run this
      // loop. First: no active position (prompt, padding), nothing to fold
      // (an empty segment is the identity of the run monoid).
      if (__ballot(qm != 0u) == 0) {
        if (kPT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pt_row[w + l4 + e] = 0.f;
            pt_row[plane + w + l4 + e] = 0.f;
            pt_row[2 * plane + w + l4 + e] = 0.f;
          }
        }
        continue;
      }
      // am[e]: lanes whose position w + 4 lane + e is active.
      uint64_t am[4], all_act = ~0ull;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        am[e] = __ballot(((qm >> (8 * e)) & 0xFFu) != 0u);
        all_act &= am[e];
      }
      const int wn = __popcll(am[0]) + __popcll(am[1]) + __popcll(am[2]) + __popcll(am[3]);
      // The differing test is on the fp32 difference y = left - right, with
      // a margin: |y| < 0.4995 implies |delta| < 0.5 in fp64; then
      // d = right - left = -y exactly. (With a tolerance instead of the
      // bitwise test, that shortcut is not taken.) Inactive positions pass
      // both tests; the shortcuts give them no contribution (a zero delta,
      // k3 and weight, which leave every sum and the maximum unchanged).
      float ys[4];
      uint64_t neq[4], differ = kBitwise ? ~0ull : 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ys[e] = vl[e] - vr[e];
        neq[e] = __ballot(__float_as_uint(vl[e]) != __float_as_uint(vr[e]));
        differ &= ~am[e] | (neq[e] & __ballot(fabsf(ys[e]) < 0.49951171875f));
      }
      // Every active position mismatches with |delta| < 0.5: straight-line
      // arithmetic (with selects when some positions are inactive), and the
      // window's active tokens form one run of mismatches.
      auto differ_fold = [&](auto masked_tag) __attribute__((always_inline)) {
        constexpr bool kM = decltype(masked_tag)::value;
        const int64_t i0 = w + l4;
        float wk = 0.f, wt = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ae = !kM || ((qm >> (8 * e)) & 0xFFu) != 0u;
          double dl = (double)vl[e] - (double)vr[e];
          if (kM) dl = ae ? dl : 0.0;
          const double ad = fabs(dl);
          asm("v_max_f64 %0, |%1|, %2" : "=v"(mx) : "v"(dl), "v"(mx));
          sa += ad;
          ss += dl;
          const float x = kM ? (ae ? -ys[e] : 0.f) : -ys[e];
          const float tx = small_tx(x);
          wk = __builtin_fmaf(tx, x, wk);
          if (kPT || !tis_count) {
            float tis = small_tis(tx, x, clip_f);
            if (kM) tis = ae ? tis : 0.f;
            wt += tis;
            if (kPT) {
              pt_row[i0 + e] = (float)ad;
              pt_row[plane + i0 + e] = tx * x;
              pt_row[2 * plane + i0 + e] = tis;
            }
          }
        }
        sk += (double)wk;
        if (!tis_count) st += (double)wt;
      };
      if (differ == ~0ull) {
        if (all_act == ~0ull) differ_fold(std::false_type{});
        else differ_fold(std::true_type{});
        mism_w += wn;
        seq = runs_combine(seq, seq_n, Runs{0, wn, wn, wn}, wn);
        seq_n += wn;
        continue;
      }
      // Every active position has identical finite scores: nothing but the
      // count (and the capped unit weights below e^0.5).
      // (The finiteness mask comes straight from the compare: a ballot of it
      // would first materialise it per lane.)
      uint64_t same = ~0ull;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        same &= ~am[e] | (~neq[e] & __builtin_amdgcn_fcmpf(fabsf(vl[e]), __builtin_inff(), 4));  // FCMP_OLT
      if (same == ~0ull) {
        if (!tis_count) {
          float wt = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) wt += ((qm >> (8 * e)) & 0xFFu) != 0u ? one_tis : 0.f;
          st += (double)wt;
        }
        if (kPT) {
          const int64_t i0 = w + l4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pt_row[i0 + e] = 0.f;
            pt_row[plane + i0 + e] = 0.f;
            pt_row[2 * plane + i0 + e] = ((qm >> (8 * e)) & 0xFFu) != 0u ? one_tis : 0.f;
          }
        }
        seq = runs_combine(seq, seq_n, Runs{-1, 0, 0, 0}, wn);
        seq_n += wn;
        continue;
      }
      unsigned amask = 0;  // bit e: position w + l4 + e is active
#pragma unroll
      for (int e = 0; e < 4; ++e) amask |= (((qm >> (8 * e)) & 0xFFu) != 0 ? 1u : 0u) << e;
      fold(w + l4, vl, vr, amask);
    }
    // Drain the repeated copies of the last windows before the kernel can
    // end (their LDS writes would otherwise land after the workgroup).
    __builtin_amdgcn_s_waitcnt(0x0F70);
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
  // once, so the order stays a fixed function of the row. With the counted
  // TIS sum, the pass also counts these tokens and sums their d.
  const double sk_small = sk;  // k3 of the tokens with |d| < 0.5
  double st2 = 0.0, sd2 = 0.0;
  int n2 = 0;
  const bool any_slow = __ballot(slow) != 0;
  if (any_slow) {
    double sk2 = 0.0;
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
        sd2 += d;
        n2 += 1;
        if (kPT) {
          pt_row[plane + i] = (float)k3;
          pt_row[2 * plane + i] = (float)tis;
        }
      }
    }
    sk += sk2;
    if (!tis_count) st += st2;
  }

  // Wave reductions; a count that is zero in every lane (the usual case for
  // the non-finite counts, and for the per-lane mismatch count when every
  // window took a shortcut) needs none.
  auto isum = [&](int v) __attribute__((always_inline)) { return __ballot(v != 0) ? wave_sum(v) : 0; };
  mism = isum(mism) + mism_w;
  nonf = isum(nonf);
  k3n = isum(k3n);
  mx = wave_max(mx);  // |delta| >= 0 and finite: fmax is the exact maximum
  sa = wave_sum(sa);
  ss = wave_sum(ss);
  sk = wave_sum(sk);
  if (tis_count) {
    // (#finite active - #|d| >= 0.5) + sum d over |d| < 0.5 + their k3 sum
    // + the capped weights of the others, in this order. Without tokens of
    // |d| >= 0.5 the terms of the others are zeros and the k3 sum is sk:
    // the same bits with three reductions fewer.
    if (any_slow) {
      const int n_small = seq_n - nonf - wave_sum(n2);
      st = (((double)n_small + (-ss - wave_sum(sd2))) + wave_sum(sk_small)) + wave_sum(st2);
    } else {
      st = ((double)(seq_n - nonf) + (-ss)) + sk;
    }
  } else {
    st = wave_sum(st);
  }

  // The 80-byte record goes out as one store instruction (lane i < 10 writes
  // its 8-byte word), not as one lane's several partial stores. The three
  // records of a sequence are adjacent (sequence-major output), so a
  // workgroup writes 240 contiguous bytes: interleaved with the streaming
  // reads, writes into three planes N records apart cost about 2 % more time
  // at large N than the same bytes in one place.
  static_assert(sizeof(lp_seq_stats) == 80, "ten 8-byte words");
  auto pack = [](int lo, int hi) __attribute__((always_inline)) {
    return (uint64_t)(uint32_t)lo | ((uint64_t)(uint32_t)hi << 32);
  };
  const uint64_t words[10] = {
      pack(seq_n, mism), pack(seq.first, seq.best), pack(nonf, k3n),
      (uint64_t)__double_as_longlong(mx), (uint64_t)__double_as_longlong(sa),
      (uint64_t)__double_as_longlong(ss), (uint64_t)__double_as_longlong(sk),
      (uint64_t)__double_as_longlong(-ss),  // sum_d: d = -delta termwise, same order
      (uint64_t)__double_as_longlong(fmin(exp(-ss), clip)),  // seq_tis
      (uint64_t)__double_as_longlong(st)};
  if (lane < 10) {
    uint64_t v = words[0];
#pragma unroll
    for (int i = 1; i < 10; ++i) v = lane == i ? words[i] : v;
    reinterpret_cast<uint64_t*>(a.out + (size_t)n * 3 + p)[lane] = v;
  }
}

}  // namespace

hipError_t launch_compare(const CompareArgs& a, hipStream_t stream) {
  const dim3 g((unsigned)a.N), b(kCompareThreads);
  const bool bitwise = a.atol < 0.0;
  const bool tis_count = a.tis_clip > 1.6487212707001282;  // e^0.5
#define LP_CMP(pt_, bw_, tc_) \
  hipLaunchKernelGGL((compare_kernel<pt_, bw_, tc_>), g, b, 0, stream, a)
  if (a.per_token) {
    if (bitwise) { if (tis_count) LP_CMP(true, true, true); else LP_CMP(true, true, false); }
    else { if (tis_count) LP_CMP(true, false, true); else LP_CMP(true, false, false); }
  } else {
    if (bitwise) { if (tis_count) LP_CMP(false, true, true); else LP_CMP(false, true, false); }
    else { if (tis_count) LP_CMP(false, false, true); else LP_CMP(false, false, false); }
  }
#undef LP_CMP
  return hipGetLastError();
}

}  // namespace lp
