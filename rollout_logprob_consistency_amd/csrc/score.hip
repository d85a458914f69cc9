// Selected-token logprob on gfx950: bf16 MFMA LM-head product, fused online
// log-sum-exp over the true vocabulary range and target gather, then a
// fixed-order merge of the per-tile partials.
//
// What is computed is the selected-token logprob of the AMD blog "Debugging
// Logprob Mismatches in LLM Reinforcement Learning" (section "Case 2: A and B
// Stay Close; C Changes": target logit minus the log-sum-exp of the whole
// vocabulary row; section "How this differs from a real temperature
// mismatch": temperature divides the logits before the normaliser), over the
// true vocabulary range named by the vime / RL-Kernel MI300X report. That
// report and the VeXact note describe batch-invariant GEMMs on other hardware;
// only the invariant is kept here, the kernel is designed for CDNA4:
//
//  * One workgroup = 4 waves computes a 352 (vocab) x 256 (token) tile of
//    Z^T = W . X^T with v_mfma_f32_16x16x32_bf16, fp32 accumulation, the whole
//    hidden dimension in ascending 32-wide MFMA steps (no split-K). Each wave
//    owns 176 x 128 outputs = 11 x 8 MFMA tiles: 256 accumulators in AGPRs
//    and 96 in VGPRs (the largest wave tile the register file holds next to
//    its fragments). Tokens are the MFMA "N" dimension: a lane holds one
//    token column and 44 vocabulary rows, so the vocabulary reduction is
//    mostly inside a lane. The 16x16x32 shape moves half as many accumulator
//    bytes per flop as 32x32x16.
//  * The chip runs this product at its power limit, so the data moved per
//    flop sets the clock: the 176 x 128 wave tile reads 14 % fewer LDS bytes
//    per flop than 128 x 128, and the 352 x 256 workgroup tile copies 14 %
//    fewer bytes from L2 into LDS.
//  * Operand stages go from HBM/L2 straight into LDS (buffer_load ... lds, no
//    VGPR round trip) through two alternating 76 KiB stage buffers (W and X
//    rows of one 64-wide K slice); the 16-byte chunks of each 128-byte row
//    are XOR-permuted so the ds_read_b128 fragment reads do not collide on
//    LDS banks. One barrier per stage; MFMAs of the previous stage's second
//    half are carried across it, and the next stage's copies are spread over
//    the whole stage.
//  * Epilogue: scale by log2(e)/temperature, mask rows >= V_true to -inf,
//    per-token max and sum of exp2 over the lane's 44 values, the lanes
//    (l, l^16, l^32, l^48) and the two vocabulary waves, in a fixed order;
//    write one (max, sum) partial per (vocabulary tile, token); the single
//    lane that holds the target logit writes it. Logits never reach memory.
//  * A second kernel merges the vocabulary tiles of each token in ascending
//    tile order and writes logprob and log-sum-exp in nats.
//
// Batch invariance: the arithmetic applied to a (token, vocabulary row) pair
// depends only on the tile shape, H and the vocabulary tile index, never on
// T, on the token's slot in its tile, on the other tokens or on which CU runs
// the tile. Rows past T or V_rows are never read from memory (the buffer
// range check; the streaming kernel clamps them) and their results are
// discarded.
#include <math.h>

#include <type_traits>

#include "lp_internal.h"

namespace lp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = kScoreTileThreads;
constexpr int kWaveV = 176;                  // vocab rows per wave
constexpr int kWaveT = 128;                  // token columns per wave
constexpr int kSubV = kWaveV / 16;           // 16-row MFMA tiles along vocab (11)
constexpr int kSubT = kWaveT / 16;           // 16-column MFMA tiles along tokens (8)
// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4],
// lgkmcnt [11:8]); only vmcnt is constrained.
constexpr int kWaitVm0 = 0x0F70;             // vmcnt(0)
constexpr int kGroupV = 4;                   // vocab tiles per scheduling group
constexpr float kLn2 = 0.693147180559945309f;

static_assert(kTileV == 2 * kWaveV && kTileT == 2 * kWaveT, "2 x 2 waves");
static_assert(kTileK == 64, "128-byte LDS rows");

// Physical 16-byte chunk of logical chunk `c` (hidden elements 8 c .. 8 c + 7
// of a 64-wide stage) in LDS row `row`. A fragment read (ds_read_b128) has
// lane l read row 16 u + (l & 15) at chunk 4 h + (l >> 4); with the chunk
// XOR-permuted by (row & 7) these reads measure SQ_LDS_BANK_CONFLICT = 0 on
// gfx950 (the permutation (row ^ (row >> 3)) & 7 measures two-way conflicts
// on every read for this pattern).
__host__ __device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// One MFMA step: 16 vocabulary rows x 16 tokens x 32 hidden elements.
__device__ __forceinline__ f32x4 mma(const bf16x8& w, const bf16x8& x, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, x, c, 0, 0, 0);
}

// Workgroup id -> (vocab tile, token tile). The hardware deals workgroups to
// the 8 XCDs round-robin; give each XCD a contiguous run of logical tiles, and
// order logical tiles in groups of kGroupV vocab tiles with the token tile
// varying fastest, so the workgroups resident on one XCD share W and X slabs
// in that XCD's L2.
__device__ __forceinline__ void tile_of(int b, int n_vt, int n_tt, int group_v, int& vt, int& tt) {
  const int G = n_vt * n_tt;
  const int xcd = b & 7, idx = b >> 3;
  const int per = G >> 3, rem = G & 7;
  const int L = (xcd < rem) ? xcd * (per + 1) + idx
                            : rem * (per + 1) + (xcd - rem) * per + idx;
  const int group = group_v * n_tt;
  const int g = L / group;
  const int first = g * group_v;
  const int gv = min(group_v, n_vt - first);
  const int r = L - g * group;
  vt = first + r % gv;
  tt = r / gv;
}

// Direct buffer -> LDS copies (buffer_load_dwordx4 ... lds): one 16-byte chunk
// per lane, the wave's 64 chunks landing contiguously at the LDS address
// (lane i at byte 16 i); no VGPR round trip.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9)

// Byte extent of a buffer resource, capped to what num_records can hold.
__device__ __forceinline__ uint32_t span_bytes(uint64_t n) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(n > 0x7FFFFFF0ull ? 0x7FFFFFF0ull : n));
}

// Buffer resource from wave-uniform values, built so the compiler keeps it in
// SGPRs (a resource it cannot prove uniform costs a waterfall loop per load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint64_t pu = ((uint64_t)hi << 32) | lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(pu), 0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// ---- Epilogue pieces shared by both tile kernels, so that a (token,
// vocabulary tile) pair goes through the same floating-point operations in the
// same order whichever kernel scores it. A wave holds kSubV MFMA tiles of 16
// vocabulary rows for each token column; `v(i, r)` returns the raw
// accumulator of vocabulary tile i, register r, for the lane's token. MFMA
// 16x16 output layout: lane l holds column (l & 15) and, in register r, row
// 4 (l >> 4) + r; the four lanes l & 15 + 16 g (g = 0..3) share a token.

// Per-token max and sum of exp2 over the wave's kWaveV rows (lanes l, l^16,
// l^32, l^48). The scale log2(e)/T is positive, so the max of the scaled
// logits is the scaled max; the scale is folded into the exp2 argument with
// one FMA. The butterfly adds the same two values in both lanes of each step,
// so all four lanes end with the same bits.
//
// kStats adds, for the entropy and the argmax, q = sum 2^d d over the same
// terms (d = scaled logit - m, log2 units; a masked row has d = -inf and adds
// nothing) and the wave-local row (0..127) of the maximum, the lowest row on
// ties (kNoRow for a wave whose rows are all masked). s and m are formed by
// exactly the same operations as without kStats.
constexpr int kNoRow = 0x7FFFFFFF;

// The value lane l ^ 16 (kOff = 16) or lane l ^ 32 (kOff = 32) holds, by the
// VALU lane swaps of gfx950 instead of an LDS permute: swapping x with itself
// puts, in the first result, the even rows' (lower half's) values into the
// odd rows (upper half) and, in the second, the odd rows' into the even rows.
template <int kOff>
__device__ __forceinline__ int xor_lane(int x) {
  const int lane = (int)__lane_id();
  if constexpr (kOff == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? (int)r[0] : (int)r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? (int)r[0] : (int)r[1];
  }
}

template <int kOff>
__device__ __forceinline__ float xor_lane(float x) {
  return __int_as_float(xor_lane<kOff>(__float_as_int(x)));
}

template <bool kStats, class Get>
__device__ __forceinline__ void wave_lse(Get v, float scale2, int lg, float& m_out, float& s_out,
                                         float& q_out, int& i_out) {
  const float NEG_INF = -__builtin_inff();
  float mr = NEG_INF;
#pragma unroll
  for (int i = 0; i < kSubV; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) mr = fmaxf(mr, v(i, r));
  int li = kNoRow;
  if (kStats) {
    // Register r of tile i holds row 16 i + 4 lg + r: rows ascend with (i, r),
    // so the last overwrite in descending order is the lowest matching row.
#pragma unroll
    for (int i = kSubV - 1; i >= 0; --i)
#pragma unroll
      for (int r = 3; r >= 0; --r) li = (v(i, r) == mr) ? 16 * i + 4 * lg + r : li;
    if (mr == NEG_INF) li = kNoRow;
  }
  auto max_step = [&](auto off_tag) __attribute__((always_inline)) {
    constexpr int kOff = decltype(off_tag)::value;
    const float mo = xor_lane<kOff>(mr);
    if (kStats) {
      const int lo = xor_lane<kOff>(li);
      li = (mo > mr) ? lo : ((mr > mo) ? li : min(li, lo));
    }
    mr = fmaxf(mr, mo);
  };
  max_step(std::integral_constant<int, 16>{});
  max_step(std::integral_constant<int, 32>{});
  const float m = mr * scale2;
  float s = 0.f, q = 0.f;
  if (mr != NEG_INF) {
    // All exponentials first, then the sums in the same order: each exp2
    // result is used well after it is formed (no wait states between them).
    float e[kSubV * 4], d[kStats ? kSubV * 4 : 1];
#pragma unroll
    for (int i = 0; i < kSubV; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float di = __builtin_fmaf(v(i, r), scale2, -m);
        e[4 * i + r] = fast_exp2(di);
        if (kStats) d[4 * i + r] = di;
      }
#pragma unroll
    for (int k = 0; k < kSubV * 4; ++k) {
      s += e[k];
      if (kStats) q = __builtin_fmaf(e[k], fmaxf(d[k], -3.0e38f), q);  // -inf row: 0 * finite
    }
  }
  s += xor_lane<16>(s);
  s += xor_lane<32>(s);
  if (kStats) {
    q += xor_lane<16>(q);
    q += xor_lane<32>(q);
  }
  m_out = m;
  s_out = s;
  q_out = q;
  i_out = li;
}

// Target gather for token t: exactly one lane of the grid holds (target, t);
// wv_lo is the first vocabulary row of the wave, lg = lane >> 4.
template <class Get>
__device__ __forceinline__ void gather_target(Get v, const ScoreArgs& a, int t, int64_t wv_lo,
                                              int lg) {
  const int64_t tgt = a.ids[t] - a.v_base;  // row of this W buffer
  const int64_t loc = tgt - wv_lo;
  if (tgt >= 0 && tgt < a.V_true && loc >= 0 && loc < kWaveV) {
    const int li = (int)loc;
    if (((li >> 2) & 3) == lg) {
      // Flat (tile, register) index of the target row; a branch-free select
      // over the lane's values picks it.
      const int k = (li >> 4) * 4 + (li & 3);
      float tv = 0.f;
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) tv = (k == i * 4 + r) ? v(i, r) : tv;
      a.tval[t] = tv * a.scale2;
    }
  }
}

// Merge of the two kWaveV-row halves of a vocabulary tile, lower half first
// (m0 is finite: row v0 < V_true lies in the lower half).
__device__ __forceinline__ void merge_halves(float m0, float s0, float m1, float s1, float& M,
                                             float& S) {
  M = fmaxf(m0, m1);
  S = __builtin_fmaf(s1, fast_exp2(m1 - M), s0 * fast_exp2(m0 - M));  // contraction spelled out
}

// Entropy term of the merge of two (max, sum, q) partials into max M: q is
// relative to each partial's max, so q_j + (m_j - M) s_j re-bases it (an
// empty partial, s_j = 0, contributes nothing even when m_j = -inf).
__device__ __forceinline__ float merge_q(float m0, float s0, float q0, float m1, float s1,
                                         float q1, float M) {
  const float t0 = s0 != 0.f ? (m0 - M) * s0 : 0.f;
  const float t1 = s1 != 0.f ? (m1 - M) * s1 : 0.f;
  return __builtin_fmaf(fast_exp2(m1 - M), q1 + t1, fast_exp2(m0 - M) * (q0 + t0));
}

// Rows at or past V_true (only in the last vocabulary tile) read as -inf:
// register r of vocabulary tile i holds row vlane + 16 i + r, vlane = first
// vocabulary row of the wave + 4 (lane >> 4). The epilogue takes this masked
// view only in that tile (a uniform branch), so the accumulators are never
// rewritten.
// The logit the epilogue uses: the fp32 accumulator, or with kBf16 that
// value rounded to bf16 (round to nearest even, v_cvt_pk_bf16_f32) and
// widened back, as an LM head whose output is stored in bf16 would give it.
template <bool kBf16>
__device__ __forceinline__ float logit(float acc) {
  if (!kBf16) return acc;
  return static_cast<float>(static_cast<__bf16>(acc));
}

#define LP_MASKED(x_, vlane_, i_, r_, V_) \
  (((vlane_) + 16 * (i_) + (r_) >= (V_)) ? -__builtin_inff() : (x_))

// One 1-KiB buffer -> LDS copy (buffer_load_dwordx4 ... lds): lane i moves 16
// bytes from rsrc + voff + soff to LDS byte address lds + 16 i. Written as
// inline assembly so that the compiler does not treat the asynchronous LDS
// write as aliasing every later LDS read (it would wait for every copy in
// flight before each read); the ring's explicit vmcnt waits and barriers order
// copies and reads instead. The LDS address goes in M0 (an operand of the
// statement); an M0 write needs one wait state before an LDS-DMA load.
__device__ __forceinline__ void copy_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, uint32_t voff,
                                         uint32_t soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
               : "memory");
}

// Stage geometry of the tile kernel: a stage is one 64-wide K slice of both
// operands, the W unit (kTileV rows of 128 bytes) followed by the X unit
// (kTileT rows); two stage buffers alternate. Wave w issues copy j of a unit
// for rows 8 (4 j + w) .. + 7.
constexpr int kRowB = kTileK * 2;               // 128 B
constexpr int kWUnitB = kTileV * kRowB;         // 44 KiB
constexpr int kXUnitB = kTileT * kRowB;         // 32 KiB
constexpr int kStageB = kWUnitB + kXUnitB;      // 76 KiB
constexpr int kCopiesW = kWUnitB / 1024 / 4;    // 1-KiB copies per wave per W unit (11)
constexpr int kCopiesX = kXUnitB / 1024 / 4;    // per X unit (8)
constexpr int kCopies = kCopiesW + kCopiesX;    // per wave per stage (19)
constexpr int kSubVA = 8;                       // vocab MFMA tiles with AGPR accumulators
constexpr int kSubVV = kSubV - kSubVA;          // ... with VGPR accumulators (3)
static_assert(kWUnitB % 4096 == 0 && kXUnitB % 4096 == 0, "whole copies per wave");
static_assert(2 * kStageB <= 160 * 1024, "LDS");
constexpr int kCopyEvery = 6;                   // MFMAs per copy across a phase
static_assert(kCopyEvery * kCopies < 2 * 8 * kSubV, "copies fit in a phase");
static_assert(kSubT == 8 && kSubVA == 8 && kSubVV <= kSubVA, "read schedule");

// The same MFMA as mma() with the accumulator in VGPRs (the AGPR file holds
// only kSubVA x kSubT accumulators). Written as assembly, so the compiler
// cannot see the MFMA's hazards; none arise: the first MFMA of an
// accumulator takes the inline constant 0 as C (mma_v0), so no VALU write
// ever precedes an MFMA read of that register; its A and B fragments are
// written only by LDS reads, which the compiler orders with lgkmcnt waits,
// and are overwritten only a whole step after their last MFMA; VALU code
// reads the accumulators only after the K loop, behind explicit wait states.
__device__ __forceinline__ void mma_v(f32x4& c, const bf16x8& w, const bf16x8& x) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(w), "v"(x));
}
__device__ __forceinline__ void mma_v0(f32x4& c, const bf16x8& w, const bf16x8& x) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(c) : "v"(w), "v"(x));
}

template <bool kStats, bool kBf16>
__global__ __launch_bounds__(kThreads, 1) void score_tile_kernel(ScoreArgs a) {
  // Two stage buffers; the 16-byte chunks of row r are XOR-permuted by
  // swz(). After the K loop the first bytes hold the cross-wave reduction.
  __shared__ __attribute__((aligned(1024))) char ring[2 * kStageB];

  int vt, tt;
  tile_of(blockIdx.x, a.n_vt, a.n_tt, kGroupV, vt, tt);
  vt = __builtin_amdgcn_readfirstlane(vt);  // uniform: keep tile state in SGPRs
  tt = __builtin_amdgcn_readfirstlane(tt);
  const int v0 = vt * kTileV, t0 = tt * kTileT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int lcol = lane & 15, lg = lane >> 4;

  // Accumulators: vocab MFMA tiles 0..7 in AGPRs, 8..10 in VGPRs. The
  // first MFMA of each starts from C = 0.
  f32x4 acc[kSubVA][kSubT], accv[kSubVV][kSubT];

  // ---- Copies. Copy j of a unit: lane i moves the 16 bytes of physical chunk
  // (i & 7) of row 8 (4 j + w) + (i >> 3), i.e. logical chunk swz(row, i & 7);
  // row & 7 = (i >> 3) & 7 for every j. The resources start at the tile's
  // first row and end at the matrix's last byte, so rows past the matrix read
  // zeros (their results are discarded); the K offset of a stage is the
  // uniform soffset, which never leaves the row.
  const char* wtile = reinterpret_cast<const char*>(a.w) + (size_t)v0 * a.H * 2;
  const char* xtile = reinterpret_cast<const char*>(a.x) + (size_t)t0 * a.ldh * 2;
  const __amdgpu_buffer_rsrc_t wres =
      make_rsrc(wtile, span_bytes((uint64_t)(a.V_rows - v0) * (uint64_t)a.H * 2));
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(
      xtile, span_bytes((uint64_t)(a.T - t0 - 1) * (uint64_t)a.ldh * 2 + (uint64_t)a.H * 2));
  const uint32_t H2 = (uint32_t)a.H * 2, X2 = (uint32_t)a.ldh * 2;
  const uint32_t lrow = (uint32_t)(8 * wave + (lane >> 3));
  const uint32_t cb = (uint32_t)(swz(lane >> 3, lane & 7) * 16);
  const uint32_t offW0 = lrow * H2 + cb, offX0 = lrow * X2 + cb;
  const uint32_t stepW = 32 * H2, stepX = 32 * X2;  // 32 rows per copy index
  const uint32_t lds0 =
      __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_char*)ring));
  const int nk = a.H / kTileK;
  // Copy c (0..18) of stage k into buffer st: c < 11 copies W rows, else X
  // rows. A stage past the end re-copies the last one (same bytes, into the
  // buffer that holds it or into one nothing reads before it is refilled).
// The per-copy row offset is added in place (an opaque add the compiler
// cannot hoist into 19 loop-invariant registers).
#define COPY(c_, k_, st_)                                                                      \
  do {                                                                                         \
    const uint32_t soff_ = (uint32_t)min((k_), nk - 1) * kRowB;                                 \
    const bool w_ = (c_) < kCopiesW;                                                           \
    const uint32_t cc_ = w_ ? (uint32_t)(c_) : (uint32_t)((c_) - kCopiesW);                     \
    uint32_t voff_;                                                                            \
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(voff_) : "s"(cc_ * (w_ ? stepW : stepX)),         \
                 "v"(w_ ? offW0 : offX0));                                                     \
    copy_lds(w_ ? wres : xres,                                                                 \
             lds0 + (uint32_t)(st_) * kStageB + (w_ ? 0u : (uint32_t)kWUnitB) + (4 * cc_ + wave) * 1024, \
             voff_, soff_);                                                                    \
  } while (0)

  // Stage 0 into buffer 0 before the first phase.
#define COPY_ALL_PROLOGUE()                                                    \
  do {                                                                         \
    _Pragma("unroll") for (int c = 0; c < kCopies; ++c) COPY(c, 0, 0);         \
  } while (0)

  // ---- Fragment reads. Fragment (tile u, half h) of an operand: lane l reads
  // row base + 16 u + (l & 15), logical chunk 4 h + (l >> 4) (hidden elements
  // 32 h + 8 (l >> 4) .. + 7 of the stage). swz() depends on the row only
  // through l & 7, so one address per (operand, half, buffer) plus an
  // immediate per tile suffice.
  uint32_t rdA[2], rdB[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int pc = swz(lcol, 4 * h + lg);
    rdA[h] = (uint32_t)((wm * kWaveV + lcol) * kRowB + pc * 16);
    rdB[h] = (uint32_t)(kWUnitB + (wn * kWaveT + lcol) * kRowB + pc * 16);
  }
  // Buffer st (0 or 1, possibly a run-time value) starts at st * kStageB.
#define RD_A(u_, h_, st_) \
  *reinterpret_cast<const bf16x8*>(ring + (rdA[(h_)] + (uint32_t)(st_) * kStageB) + (u_) * 2048)
#define RD_B(u_, h_, st_) \
  *reinterpret_cast<const bf16x8*>(ring + (rdB[(h_)] + (uint32_t)(st_) * kStageB) + (u_) * 2048)
#define FENCE() __builtin_amdgcn_sched_barrier(0)

  // W fragments of MFMA groups 0..7 are single-buffered: fa[g] is reloaded
  // with the next step's fragment right after group g has used it. Those of
  // groups 8..10 (the VGPR-accumulator groups, last in a step) and the X
  // fragments alternate between two buffers, so every read of a step is
  // issued at least 24 MFMAs before the step ends.
  bf16x8 fa[kSubVA], fx0[kSubVV], fx1[kSubVV], fb0[kSubT], fb1[kSubT];

  // One step = kSubV groups of 8 MFMAs (W tile g with X tiles 0..7), 32
  // hidden elements, on (fa, mx_, mb_) (skipped with do_mma_ false); reads
  // of the next step's fragments from (half rh_, buffer rs_): X tile i into
  // rb_ after the 4th MFMA of group i, W tile g < 8 into fa[g] after group
  // g, W tile 8 + i into rx_ after the 6th MFMA of group i. A phase (two
  // steps, p0_ = 0 or 8 kSubV) issues copy c of stage ck_ into buffer cs_
  // after its MFMA slot kCopyEvery c + 1. The order is fixed instruction by
  // instruction.
#define STEP(do_mma_, z_, do_rd_, mx_, mb_, rx_, rb_, rh_, rs_, p0_, ck_, cs_)       \
  do {                                                                             \
    _Pragma("unroll") for (int u = 0; u < 8 * kSubV; ++u) {                        \
      const int g_ = u >> 3, b_ = u & 7;                                           \
      if (do_mma_) {                                                               \
        if (g_ < kSubVA) {                                                         \
          const int ga_ = g_ < kSubVA ? g_ : 0;                                    \
          acc[ga_][b_] = mma(fa[ga_], mb_[b_], (z_) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[ga_][b_]); \
        } else {                                                                   \
          const int gv_ = g_ >= kSubVA ? g_ - kSubVA : 0;                          \
          if (z_) mma_v0(accv[gv_][b_], mx_[gv_], mb_[b_]);                        \
          else mma_v(accv[gv_][b_], mx_[gv_], mb_[b_]);                            \
        }                                                                          \
      }                                                                            \
      if ((do_rd_) && b_ == 3 && g_ < kSubT) rb_[g_ < kSubT ? g_ : 0] = RD_B(g_, (rh_), (rs_)); \
      if ((do_rd_) && b_ == 5 && g_ < kSubVV) rx_[g_ < kSubVV ? g_ : 0] =                      \
          RD_A(kSubVA + g_, (rh_), (rs_));                                         \
      if ((do_rd_) && b_ == 7 && g_ < kSubVA) fa[g_ < kSubVA ? g_ : 0] = RD_A(g_, (rh_), (rs_)); \
      {                                                                            \
        const int pu_ = (p0_) + u;                                                 \
        if (pu_ % kCopyEvery == 1 && pu_ / kCopyEvery < kCopies)                   \
          COPY(pu_ / kCopyEvery, (ck_), (cs_));                                    \
      }                                                                            \
      FENCE();                                                                     \
    }                                                                              \
  } while (0)

  // Phase k: once stage k has landed (its copies were issued during phase
  // k - 1) and every wave has finished reading stage k - 1, one barrier;
  // then the first step runs the MFMAs of stage k - 1's second half (their
  // fragments were read during phase k - 1) while reading stage k's first
  // half, and the second step runs stage k's first half while reading its
  // second half. Stage k + 1 is copied, across the whole phase, into the
  // buffer stage k - 1 has left.
  COPY_ALL_PROLOGUE();
  // Phase 0 has no carried MFMAs.
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __syncthreads();
  FENCE();
  STEP(false, false, true, fx1, fb1, fx0, fb0, 0, 0, 0, 1, 1);
  STEP(true, true, true, fx0, fb0, fx1, fb1, 1, 0, 8 * kSubV, 1, 1);
  for (int k = 1; k < nk; ++k) {
    const int sb = k & 1;
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    FENCE();
    STEP(true, false, true, fx1, fb1, fx0, fb0, 0, sb, 0, k + 1, sb ^ 1);
    STEP(true, false, true, fx0, fb0, fx1, fb1, 1, sb, 8 * kSubV, k + 1, sb ^ 1);
  }
  STEP(true, false, false, fx1, fb1, fx0, fb0, 0, 0, 2 * 8 * kSubV, 0, 0);  // stage nk - 1's second half
  // Drain the tail copies and reads before the LDS is reused; the wait
  // states cover the VALU reads of the VGPR accumulators.
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // Empty statements that claim to rewrite each VGPR accumulator: every later
  // read of one is ordered after the wait states above (a plain asm is a
  // fence for memory only, not for register-to-register code).
#pragma unroll
  for (int i = 0; i < kSubVV; ++i)
#pragma unroll
    for (int j = 0; j < kSubT; ++j) asm volatile("" : "+v"(accv[i][j]));
  // bf16-logit mode: round every accumulator once, in place, so that the
  // epilogue below holds no second copy of the logits.
  if (kBf16) {
#pragma unroll
    for (int j = 0; j < kSubT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int i = 0; i < kSubVA; ++i) acc[i][j][r] = logit<true>(acc[i][j][r]);
#pragma unroll
        for (int i = 0; i < kSubVV; ++i) accv[i][j][r] = logit<true>(accv[i][j][r]);
      }
  }
#undef STEP
#undef COPY
#undef RD_A
#undef RD_B
#undef FENCE
  float (*red_m)[kTileT] = reinterpret_cast<float (*)[kTileT]>(ring);
  float (*red_s)[kTileT] = reinterpret_cast<float (*)[kTileT]>(ring + 2 * kTileT * sizeof(float));
  float (*red_q)[kTileT] = reinterpret_cast<float (*)[kTileT]>(ring + 4 * kTileT * sizeof(float));
  int (*red_i)[kTileT] = reinterpret_cast<int (*)[kTileT]>(ring + 6 * kTileT * sizeof(float));

  // ---- Epilogue: per-token online LSE over this wave's kWaveV vocab rows. ----
  // Without the statistics, the lane-derived indices are formed again from a
  // lane id that a volatile asm produces (the compiler cannot merge it with
  // the prologue's), so none of the prologue's per-lane values stays live
  // across the K loop, where every VGPR is taken (they would be spilled). The
  // statistics variants keep the prologue's values: with theirs, the
  // allocation that results passes the MFMA hazard check.
  int lane_e = lane;
  if (!kStats)
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int tid_e = kStats ? tid : wave * 64 + lane_e;
  const int lcol_e = kStats ? lcol : lane_e & 15, lg_e = kStats ? lg : lane_e >> 4;
  const int vlane = v0 + wm * kWaveV + 4 * lg_e;
  const bool vtail = v0 + kTileV > a.V_true;
  const int64_t wv_lo = v0 + wm * kWaveV;

#pragma unroll
  for (int j = 0; j < kSubT; ++j) {
    const int tl = wn * kWaveT + j * 16 + lcol_e;
    const int t = t0 + tl;
    auto raw = [&](int i, int r) __attribute__((always_inline)) {
      return i < kSubVA ? acc[i < kSubVA ? i : 0][j][r] : accv[i >= kSubVA ? i - kSubVA : 0][j][r];
    };
    auto v = [&](int i, int r) __attribute__((always_inline)) { return raw(i, r); };
    auto vm = [&](int i, int r) __attribute__((always_inline)) {
      return LP_MASKED(raw(i, r), vlane, i, r, a.V_true);
    };
    float m, s, q;
    int li;
    if (vtail) wave_lse<kStats>(vm, a.scale2, lg_e, m, s, q, li);
    else wave_lse<kStats>(v, a.scale2, lg_e, m, s, q, li);
    if (t < a.T) gather_target(v, a, t, wv_lo, lg_e);  // targets lie below V_true
    if (lg_e == 0) {
      red_m[wm][tl] = m;
      red_s[wm][tl] = s;
      if (kStats) {
        red_q[wm][tl] = q;
        red_i[wm][tl] = li == kNoRow ? kNoRow : a.v_base + (int)wv_lo + li;
      }
    }
  }
  __syncthreads();

  {
    const int tl = tid_e;
    const int t = t0 + tl;
    float M, S;
    merge_halves(red_m[0][tl], red_s[0][tl], red_m[1][tl], red_s[1][tl], M, S);
    if (t < a.T) {
      a.part_m[(size_t)vt * a.T + t] = M;
      a.part_s[(size_t)vt * a.T + t] = S;
      if (kStats) {
        a.part_q[(size_t)vt * a.T + t] = merge_q(red_m[0][tl], red_s[0][tl], red_q[0][tl],
                                                 red_m[1][tl], red_s[1][tl], red_q[1][tl], M);
        // The lower half wins ties: its rows come first.
        a.part_i[(size_t)vt * a.T + t] = red_m[1][tl] > red_m[0][tl] ? red_i[1][tl] : red_i[0][tl];
      }
    }
  }
}

// ---- Streaming kernels for small batches (HBM-bound on W). ----
// With few rows the product is a stream over W (2 V H bytes) and the 352 x 256
// tiles would be mostly padding. Here a work item is one 176-row half of a
// vocabulary tile x a few 16-token MFMA tiles, computed by a single wave in
// exactly the placement of the 352 x 256 kernel -- vocabulary row -> (MFMA
// tile i, lane group, register), token -> MFMA column, the same
// v_mfma_f32_16x16x32_bf16 chain over 32-wide K steps in ascending order --
// and the same per-wave epilogue (wave_lse), so every row's bits match. The
// wave writes its half's (max, sum) partial; the merge kernel applies
// merge_halves before folding the tiles, as the 352 x 256 kernel does in LDS.
//
// score_stream_kernel (items of 16 or 32 tokens): one wave per item and one
// item per wave, so the items of a batch (864 at the 151 936-row vocabulary)
// all run at once, one wave per SIMD, and none is left with a second item
// after the others finish. Each lane loads its MFMA fragments straight from
// HBM into registers -- 16 bytes of one W row and of one token row per
// 32-wide chunk, the two 64-byte halves of each row's 128-byte segment back
// to back -- with the next 64-wide K stage (22.5 KiB of W per wave) in flight
// while the current one is multiplied. Measured at the Qwen3-8B head, deeper
// rings (three stages) and smaller or larger bursts per row run no faster:
// one-wave-per-item streams of this shape top out near 5.9 TB/s on MI355X
// (a plain sweep of the same bytes reaches 7 TB/s), and the kernel is within
// about 12 % of that.
template <int NT>
struct Stream {
  static constexpr int kTok = 16 * NT;  // tokens per item
  static constexpr int kTilesB = NT;    // 16-token MFMA tiles
  static constexpr int kRing = 2;       // 64-wide K stages in registers
};

template <int NT, bool kStats, bool kBf16>
__global__ __launch_bounds__(64) void score_stream_kernel(ScoreArgs a, int n_items) {
  using S = Stream<NT>;
  constexpr int R = S::kRing;
  const int L = blockIdx.x;
  if (L >= n_items) return;
  const int lane = threadIdx.x, lcol = lane & 15, lg = lane >> 4;
  const int nk = a.H / kTileK;
  const uint32_t H2 = (uint32_t)a.H * 2, X2 = (uint32_t)a.ldh * 2;
  const int vh = L / a.n_tt, tt = L - vh * a.n_tt;
  // vh = 2 vt + half. The resource starts at the tile's first row v0 <
  // V_rows; rows are clamped to the matrix (the upper half of the last tile
  // may lie wholly past V_rows), results there are discarded.
  const int v0 = (vh >> 1) * kTileV, t0 = tt * S::kTok;
  const __amdgpu_buffer_rsrc_t wres =
      make_rsrc(reinterpret_cast<const char*>(a.w) + (size_t)v0 * H2,
                span_bytes((uint64_t)(a.V_rows - v0) * H2));
  const __amdgpu_buffer_rsrc_t xres =
      make_rsrc(reinterpret_cast<const char*>(a.x) + (size_t)t0 * X2,
                span_bytes((uint64_t)(a.T - t0 - 1) * X2 + H2));
  const int vr0 = (vh & 1) * kWaveV, vmax = a.V_rows - 1 - v0, tmax = a.T - 1 - t0;
  // Lane l holds row 16 i + (l & 15) (W) or token 16 jj + (l & 15) (X),
  // hidden elements 32 c + 8 (l >> 4) .. + 7 of each stage's chunk c.
  uint32_t woff[kSubV], xoff[S::kTilesB];
#pragma unroll
  for (int i = 0; i < kSubV; ++i) woff[i] = (uint32_t)min(vr0 + 16 * i + lcol, vmax) * H2 + 16 * lg;
#pragma unroll
  for (int jj = 0; jj < S::kTilesB; ++jj) xoff[jj] = (uint32_t)min(16 * jj + lcol, tmax) * X2 + 16 * lg;

  bf16x8 fw[R][2][kSubV], fx[R][2][S::kTilesB];
  auto ld = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
  };
  // Loads of stage k, clamped to the last stage: the ring's final refills
  // re-read it, so every iteration issues the same loads and the compiler's
  // wait counts stay exact.
  auto issue = [&](bf16x8 (&w)[2][kSubV], bf16x8 (&x)[2][S::kTilesB], int k)
      __attribute__((always_inline)) {
    const int soff = min(k, nk - 1) * (kTileK * 2);
#pragma unroll
    for (int i = 0; i < kSubV; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) w[c][i] = ld(wres, woff[i] + 64 * c, soff);
#pragma unroll
    for (int jj = 0; jj < S::kTilesB; ++jj)
#pragma unroll
      for (int c = 0; c < 2; ++c) x[c][jj] = ld(xres, xoff[jj] + 64 * c, soff);
  };
  f32x4 acc[kSubV][S::kTilesB];
  auto compute = [&](bf16x8 (&w)[2][kSubV], bf16x8 (&x)[2][S::kTilesB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
#pragma unroll
        for (int jj = 0; jj < S::kTilesB; ++jj) acc[i][jj] = mma(w[c][i], x[c][jj], acc[i][jj]);
  };

#pragma unroll
  for (int i = 0; i < kSubV; ++i)
#pragma unroll
    for (int jj = 0; jj < S::kTilesB; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][jj][r] = 0.f;
#pragma unroll
  for (int u = 0; u < R - 1; ++u) issue(fw[u], fx[u], u);
  int k0 = 0;
  for (; k0 + R <= nk; k0 += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      // Stage k0 + u + R - 1 goes into the slot stage k0 + u - 1 has left.
      issue(fw[(u + R - 1) % R], fx[(u + R - 1) % R], k0 + u + R - 1);
      // Keep the refill ahead of this stage's MFMAs: left alone, the
      // scheduler sinks each load down to its first use and waits for it.
      __builtin_amdgcn_sched_barrier(0);
      compute(fw[u], fx[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // The last nk - k0 < R stages sit in slots 0 .. nk - k0 - 1 already.
#pragma unroll
  for (int u = 0; u < R - 1; ++u)
    if (k0 + u < nk) compute(fw[u], fx[u]);

  const int vbase = vh * kWaveV;
  const int vlane = vbase + 4 * lg;
  const bool vtail = vbase + kWaveV > a.V_true;
#pragma unroll
  for (int jj = 0; jj < S::kTilesB; ++jj) {
    const int t = t0 + 16 * jj + lcol;
    auto v = [&](int i, int r) __attribute__((always_inline)) {
      return logit<kBf16>(acc[i][jj][r]);
    };
    auto vm = [&](int i, int r) __attribute__((always_inline)) {
      return LP_MASKED(logit<kBf16>(acc[i][jj][r]), vlane, i, r, a.V_true);
    };
    float m, s, q;
    int li;
    if (vtail) wave_lse<kStats>(vm, a.scale2, lg, m, s, q, li);
    else wave_lse<kStats>(v, a.scale2, lg, m, s, q, li);
    if (t < a.T) {
      gather_target(v, a, t, vbase, lg);  // targets lie below V_true
      if (lg == 0) {
        a.part_m[(size_t)vh * a.T + t] = m;
        a.part_s[(size_t)vh * a.T + t] = s;
        if (kStats) {
          a.part_q[(size_t)vh * a.T + t] = q;
          a.part_i[(size_t)vh * a.T + t] = li == kNoRow ? kNoRow : a.v_base + vbase + li;
        }
      }
    }
  }
}

// score_stream_lds_kernel (items of 64 tokens): the 176 x 64 accumulators
// leave no registers for a ring of W fragments, so the stages go through LDS.
// The grid is persistent (a fixed number of one-wave workgroups per CU, each
// taking items b, b + G, b + 2G, ... with XCD-contiguous numbering, token
// tiles fastest so the waves of one XCD that share a W half-tile run
// together). Each wave streams its items' 64-wide K stages (128-byte row
// segments of W) through a ring of two LDS slots with direct buffer -> LDS
// copies, one stage in flight, continuing across item boundaries; being alone
// in its workgroup, a wave only waits on its own vmcnt, never on a barrier;
// as many waves per CU as the LDS holds.
constexpr int kSmK = kTileK;                   // hidden elements per stage
constexpr int kSmRowB = kSmK * 2;              // LDS row bytes (128)
constexpr int kSmNC = kSmRowB / 16;            // 16-byte chunks per row (8)
constexpr int kSmRPC = 1024 / kSmRowB;         // rows per 1-KiB wave copy (8)
constexpr int kSmRowsA = kWaveV;               // 176 W rows per item
constexpr int kSmCopiesA = kSmRowsA * kSmRowB / 1024;

template <int ST>
struct StreamLds {
  static constexpr int kTok = 32 * ST;                     // tokens per item
  static constexpr int kTilesB = 2 * ST;                   // 16-token MFMA tiles
  static constexpr int kCopiesB = kTok * kSmRowB / 1024;   // 4 ST
  static constexpr int kCopies = kSmCopiesA + kCopiesB;    // per stage
  static constexpr int kSlotA = kSmRowsA * kSmRowB;        // 22 KiB
  static constexpr int kSlotB = kTok * kSmRowB;            // 4 ST KiB
  static constexpr int kSlot = kSlotA + kSlotB;
  // Two 30 KiB stages and two waves per CU (three stages would leave one wave
  // per CU, measured 70 % slower).
  static constexpr int kStages = 2;
  static constexpr int kLds = kStages * kSlot;
  static_assert((kStages - 1) * kCopies <= 63, "vmcnt holds at most 63");
};

template <int ST, bool kStats, bool kBf16>
__global__ __launch_bounds__(64) void score_stream_lds_kernel(ScoreArgs a, int n_items) {
  using S = StreamLds<ST>;
  __shared__ __attribute__((aligned(1024))) char ring[S::kLds];
  const int lane = threadIdx.x;
  const int G = gridDim.x;  // a multiple of 8
  const int xb = (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
  const int nk = a.H / kSmK;
  const int n_mine = xb < n_items ? (n_items - xb + G - 1) / G : 0;
  const int n_stages = n_mine * nk;
  const uint32_t H2 = (uint32_t)a.H * 2, X2 = (uint32_t)a.ldh * 2;
  // Copy lane mapping: copy q fills rows kSmRPC q .. + kSmRPC - 1; lane i
  // writes physical chunk i % kSmNC of row kSmRPC q + i / kSmNC, i.e. the
  // logical chunk swz(row, i % kSmNC) (the permutation is an involution).
  const int lrow = lane / kSmNC;
#define SM_LC(q_) ((uint32_t)(swz(kSmRPC * (q_) + lrow, lane % kSmNC) * 16))

  // Enqueue the copies of flat stage g (item g / nk, K stage g % nk).
  auto issue = [&](int g) __attribute__((always_inline)) {
    const int it = g / nk, kt = g - it * nk;
    const int L = xb + it * G;
    const int vh = L / a.n_tt, tt = L - vh * a.n_tt;
    // vh = 2 vt + half. The resource starts at the tile's first row v0 <
    // V_rows; rows are clamped to the matrix (the upper half of the last
    // tile may lie wholly past V_rows), results there are discarded.
    const int v0 = (vh >> 1) * kTileV, t0 = tt * S::kTok;
    const __amdgpu_buffer_rsrc_t wres =
        make_rsrc(reinterpret_cast<const char*>(a.w) + (size_t)v0 * H2,
                  span_bytes((uint64_t)(a.V_rows - v0) * H2));
    const __amdgpu_buffer_rsrc_t xres =
        make_rsrc(reinterpret_cast<const char*>(a.x) + (size_t)t0 * X2,
                  span_bytes((uint64_t)(a.T - t0 - 1) * X2 + H2));
    lds_char* slot = (lds_char*)ring + (g % S::kStages) * S::kSlot;
    const int koff = kt * kSmRowB;
    const int vr0 = (vh & 1) * kWaveV, vmax = a.V_rows - 1 - v0, tmax = a.T - 1 - t0;
#pragma unroll
    for (int q = 0; q < kSmCopiesA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wres, (lds_void*)(slot + q * 1024), 16,
          (uint32_t)min(vr0 + kSmRPC * q + lrow, vmax) * H2 + SM_LC(q), koff, 0, 0);
#pragma unroll
    for (int q = 0; q < S::kCopiesB; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (lds_void*)(slot + S::kSlotA + q * 1024), 16,
          (uint32_t)min(kSmRPC * q + lrow, tmax) * X2 + SM_LC(q), koff, 0, 0);
  };

  // Fragment reads: row 16 i + (l & 15) of the half-tile (W) or 16 jj +
  // (l & 15) of the token tile (X), logical chunk 4 h + (l >> 4).
  const int lcol = lane & 15, lg = lane >> 4;
#define SM_RD(row0_, h_) \
  ((uint32_t)(((row0_) + lcol) * kSmRowB + swz((row0_) + lcol, 4 * (h_) + lg) * 16))

  f32x4 acc[kSubV][S::kTilesB];
  for (int g = 0; g < S::kStages - 1 && g < n_stages; ++g) issue(g);
  for (int g = 0; g < n_stages; ++g) {
    if (g + S::kStages - 1 < n_stages) {
      issue(g + S::kStages - 1);
      // Stage g has landed once at most (kStages - 1) stages' copies remain.
      __builtin_amdgcn_s_waitcnt(0x0F70 | (((S::kStages - 1) * S::kCopies) & 15) |
                                 ((((S::kStages - 1) * S::kCopies) >> 4) << 14));
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    const int kt = g % nk;
    if (kt == 0) {
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
#pragma unroll
        for (int jj = 0; jj < S::kTilesB; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][jj][r] = 0.f;
    }
    const char* slot = ring + (g % S::kStages) * S::kSlot;
#pragma unroll
    for (int h = 0; h < kSmK / 32; ++h) {
      bf16x8 fa[kSubV], fb[S::kTilesB];
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(slot + SM_RD(16 * i, h));
#pragma unroll
      for (int jj = 0; jj < S::kTilesB; ++jj)
        fb[jj] = *reinterpret_cast<const bf16x8*>(slot + S::kSlotA + SM_RD(16 * jj, h));
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
#pragma unroll
        for (int jj = 0; jj < S::kTilesB; ++jj) acc[i][jj] = mma(fa[i], fb[jj], acc[i][jj]);
    }
    if (kt == nk - 1) {
      const int L = xb + (g / nk) * G;
      const int vh = L / a.n_tt, tt = L - vh * a.n_tt;
      const int vbase = vh * kWaveV, t0 = tt * S::kTok;
      const int vlane = vbase + 4 * lg;
      const bool vtail = vbase + kWaveV > a.V_true;
#pragma unroll
      for (int jj = 0; jj < S::kTilesB; ++jj) {
        const int t = t0 + 16 * jj + lcol;
        auto v = [&](int i, int r) __attribute__((always_inline)) {
          return logit<kBf16>(acc[i][jj][r]);
        };
        auto vm = [&](int i, int r) __attribute__((always_inline)) {
          return LP_MASKED(logit<kBf16>(acc[i][jj][r]), vlane, i, r, a.V_true);
        };
        float m, s, q;
        int li;
        if (vtail) wave_lse<kStats>(vm, a.scale2, lg, m, s, q, li);
        else wave_lse<kStats>(v, a.scale2, lg, m, s, q, li);
        if (t < a.T) {
          gather_target(v, a, t, vbase, lg);  // targets lie below V_true
          if (lg == 0) {
            a.part_m[(size_t)vh * a.T + t] = m;
            a.part_s[(size_t)vh * a.T + t] = s;
            if (kStats) {
              a.part_q[(size_t)vh * a.T + t] = q;
              a.part_i[(size_t)vh * a.T + t] = li == kNoRow ? kNoRow : a.v_base + vbase + li;
            }
          }
        }
      }
    }
  }
}

#undef SM_LC
#undef SM_RD

// Merge of the per-tile partials. A workgroup takes 64 consecutive tokens
// (one per lane, so every partial row is read coalesced) and kMergeSegs
// waves; wave w folds the vocabulary tiles of segment w in ascending order,
// then the segment results are folded in segment order. Segment bounds depend
// only on the number of vocabulary tiles, so the order is the same for every
// batch.

__device__ __forceinline__ void lse_fold(float& M, float& S, float m, float s) {
  const float Mn = fmaxf(M, m);
  // exp2(-inf) = 0 on first use; the contraction is spelled out.
  S = __builtin_fmaf(s, fast_exp2(m - Mn), S * fast_exp2(M - Mn));
  M = Mn;
}

// The same fold with the entropy term q and the argmax i carried along; an
// equal maximum keeps the earlier (lower) index.
__device__ __forceinline__ void lse_fold_stats(float& M, float& S, float& Q, int& I, float m,
                                               float s, float q, int i) {
  const float Mn = fmaxf(M, m);
  Q = merge_q(M, S, Q, m, s, q, Mn);
  I = m > M ? i : I;
  S = __builtin_fmaf(s, fast_exp2(m - Mn), S * fast_exp2(M - Mn));
  M = Mn;
}

// Fold of the vocabulary tiles [lo, hi) (indices of the partial planes) of
// one merge segment for token t, in ascending order, from the empty partial.
// kHalves: the partials are per 176-row half of each vocabulary tile (rows
// 2 vt and 2 vt + 1), merged with merge_halves first. kStats: the entropy
// term and the argmax are carried along. The partials of kB tiles are loaded
// before any of them is folded (the fold is a dependent chain; loaded one
// tile at a time, a one-row merge waited a memory round trip per tile);
// loads past hi repeat tile hi - 1 and are not folded.
template <bool kHalves, bool kStats>
__device__ __forceinline__ void seg_fold(const ScoreArgs& a, int t, int lo, int hi, float& M,
                                         float& S, float& Q, int& I) {
  M = -__builtin_inff();
  S = 0.f;
  Q = 0.f;
  I = kNoRow;
  const float* pm = a.part_m + t;
  const float* ps = a.part_s + t;
  const float* pq = a.part_q + t;
  const int* pi = a.part_i + t;
  constexpr int kP = kHalves ? 2 : 1;  // partial rows per tile
  constexpr int kB = kStats ? 8 : 16;  // tiles per block of loads
  for (int v0 = lo; v0 < hi; v0 += kB) {
    float bm[kB][kP], bs[kB][kP], bq[kStats ? kB : 1][kP];
    int bi[kStats ? kB : 1][kP];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int vt = min(v0 + j, hi - 1);
#pragma unroll
      for (int h = 0; h < kP; ++h) {
        const size_t r = (size_t)(kP * vt + h) * a.T;
        bm[j][h] = pm[r];
        bs[j][h] = ps[r];
        if (kStats) {
          bq[kStats ? j : 0][h] = pq[r];
          bi[kStats ? j : 0][h] = pi[r];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (v0 + j >= hi) continue;  // uniform: past the segment
      const int js = kStats ? j : 0;
      if (kHalves) {
        float m, s;
        merge_halves(bm[j][0], bs[j][0], bm[j][1], bs[j][1], m, s);
        if (kStats) {
          const float q = merge_q(bm[j][0], bs[j][0], bq[js][0], bm[j][1], bs[j][1], bq[js][1], m);
          const int i = bm[j][1] > bm[j][0] ? bi[js][1] : bi[js][0];
          lse_fold_stats(M, S, Q, I, m, s, q, i);
        } else {
          lse_fold(M, S, m, s);
        }
      } else {
        if (kStats) lse_fold_stats(M, S, Q, I, bm[j][0], bs[j][0], bq[js][0], bi[js][0]);
        else lse_fold(M, S, bm[j][0], bs[j][0]);
      }
    }
  }
}

// Outputs of row t from its fully folded (M, S[, Q, I]) and its scaled
// target logit tv (ok: the target id lies in [0, V_true)).
template <bool kStats>
__device__ __forceinline__ void finish_row(const ScoreArgs& a, int t, float M, float S, float Q,
                                           int I, float tv, bool ok) {
  const float l2s = fast_log2(S);
  const float lse2 = M + l2s;
  a.out_lp[t] = ok ? (tv - lse2) * kLn2 : __builtin_nanf("");
  if (a.out_lse) a.out_lse[t] = lse2 * kLn2;
  if (kStats) {
    // H = ln 2 (log2 S - Q / S): the log-sum-exp minus the mean scaled logit.
    a.out_ent[t] = (l2s - Q / S) * kLn2;
    a.out_argmax[t] = I;
  }
  if (!ok && a.bad_rows) atomicAdd(a.bad_rows, 1);
}

template <bool kHalves, bool kStats>
__global__ __launch_bounds__(64 * kMergeSegs) void lse_merge_kernel(ScoreArgs a) {
  __shared__ float seg_m[kMergeSegs][64];
  __shared__ float seg_s[kMergeSegs][64];
  __shared__ float seg_q[kStats ? kMergeSegs : 1][64];
  __shared__ int seg_i[kStats ? kMergeSegs : 1][64];
  const int lane = threadIdx.x & 63, seg = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + lane;
  const int per = (a.n_vt + kMergeSegs - 1) / kMergeSegs;
  const int lo = min(a.n_vt, seg * per), hi = min(a.n_vt, lo + per);
  float M = -__builtin_inff(), S = 0.f, Q = 0.f;
  int I = kNoRow;
  if (t < a.T) seg_fold<kHalves, kStats>(a, t, lo, hi, M, S, Q, I);
  seg_m[seg][lane] = M;
  seg_s[seg][lane] = S;
  if (kStats) {
    seg_q[seg][lane] = Q;
    seg_i[seg][lane] = I;
  }
  __syncthreads();
  if (seg != 0 || t >= a.T) return;
  M = seg_m[0][lane];
  S = seg_s[0][lane];
  if (kStats) {
    Q = seg_q[0][lane];
    I = seg_i[0][lane];
  }
#pragma unroll
  for (int g = 1; g < kMergeSegs; ++g) {  // an empty segment (-inf, 0) folds to a no-op
    if (kStats) lse_fold_stats(M, S, Q, I, seg_m[g][lane], seg_s[g][lane], seg_q[g][lane], seg_i[g][lane]);
    else lse_fold(M, S, seg_m[g][lane], seg_s[g][lane]);
  }
  const int64_t id = a.ids[t];
  const bool ok = id >= 0 && id < a.V_true;
  finish_row<kStats>(a, t, M, S, Q, I, ok ? a.tval[t] : 0.f, ok);
}

// ---- Vocabulary-parallel scoring. ----
// A shard owns whole merge segments (the segment bounds above, fixed by the
// true vocabulary size alone). It scores its rows with the kernels above
// (same tiles, same K order, same epilogue) and folds each of its segments
// exactly as lse_merge_kernel does; after the records of all segments are
// gathered, shard_merge_kernel folds them in segment order as
// lse_merge_kernel's second stage does. Every float operation and its order
// are those of the one-buffer path, so the results are bitwise equal.
//
// Record of segment g: s.F planes of T floats at s.out + g F T -- max, sum,
// target logit (0 unless the target row lies in the segment), and with stats
// the entropy term and the argmax (int32 bits).
template <bool kHalves, bool kStats>
__global__ __launch_bounds__(64) void shard_fold_kernel(ScoreArgs a, ShardArgs s) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  if (t >= a.T) return;
  const int g = s.seg_lo + blockIdx.y;
  const int lo = min(s.n_vt_glob, g * s.per), hi = min(s.n_vt_glob, lo + s.per);
  float M, S, Q;
  int I;
  seg_fold<kHalves, kStats>(a, t, lo - s.tile_base, hi - s.tile_base, M, S, Q, I);
  const int64_t id = a.ids[t];
  const int64_t r0 = (int64_t)lo * kTileV, r1 = min((int64_t)hi * kTileV, (int64_t)s.V_true_glob);
  float* rec = s.out + (size_t)g * s.F * a.T + t;
  rec[0] = M;
  rec[(size_t)a.T] = S;
  rec[2 * (size_t)a.T] = (id >= r0 && id < r1) ? a.tval[t] : 0.f;
  if (kStats) {
    rec[3 * (size_t)a.T] = Q;
    reinterpret_cast<int*>(rec)[4 * (size_t)a.T] = I;
  }
}

template <bool kStats>
__global__ __launch_bounds__(256) void shard_merge_kernel(ScoreArgs a, ShardArgs s) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  const size_t T = (size_t)a.T, FT = (size_t)s.F * T;
  const float* rec = s.out + t;
  float M = rec[0], S = rec[T], Q = 0.f;
  int I = kNoRow;
  if (kStats) {
    Q = rec[3 * T];
    I = reinterpret_cast<const int*>(rec)[4 * T];
  }
#pragma unroll
  for (int g = 1; g < kMergeSegs; ++g) {
    const float* r = rec + g * FT;
    if (kStats) lse_fold_stats(M, S, Q, I, r[0], r[T], r[3 * T], reinterpret_cast<const int*>(r)[4 * T]);
    else lse_fold(M, S, r[0], r[T]);
  }
  const int64_t id = a.ids[t];
  const bool ok = id >= 0 && id < a.V_true;
  float tv = 0.f;
  if (ok) tv = rec[(size_t)((int)(id / kTileV) / s.per) * FT + 2 * T];
  finish_row<kStats>(a, t, M, S, Q, I, tv, ok);
}

}  // namespace

// Streaming kernel choice: 16-token MFMA tiles per item (1, 2: the register
// kernel; 4: the LDS kernel); 0 = the 352 x 256 kernel.
static int stream_tokens(int64_t T) {
  if (T <= 16) return 1;
  if (T <= 32) return 2;
  if (T <= kSkinnyMaxT) return 4;
  return 0;
}

ScoreWorkspace score_workspace_layout(int64_t T, int64_t V_true, bool stats) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t n_vt = (size_t)((V_true + kTileV - 1) / kTileV);
  const size_t rows = stream_tokens(T) ? 2 * n_vt : n_vt;  // half-tile partials
  const size_t plane = rows * (size_t)T * sizeof(float);
  ScoreWorkspace w;
  w.off_m = 0;
  w.off_s = up(w.off_m + plane);
  w.off_t = up(w.off_s + plane);
  w.off_q = up(w.off_t + (size_t)T * sizeof(float));
  w.off_i = stats ? up(w.off_q + plane) : w.off_q;
  w.total = stats ? up(w.off_i + plane) : w.off_q;
  return w;
}

template <int NT, bool kStats, bool kBf16>
static void launch_stream(ScoreArgs a, hipStream_t stream) {
  a.n_tt = (a.T + 16 * NT - 1) / (16 * NT);
  const int n_items = 2 * a.n_vt * a.n_tt;
  if constexpr (NT <= 2) {  // one wave (and workgroup) per item
    hipLaunchKernelGGL((score_stream_kernel<NT, kStats, kBf16>), dim3(n_items), dim3(64), 0,
                       stream, a, n_items);
  } else {
    // Workgroups (one wave each) per CU: as many as the LDS ring allows.
    constexpr int ST = NT / 2;
    const int per_cu = (160 * 1024) / StreamLds<ST>::kLds;
    const int grid = 256 * (per_cu < 8 ? per_cu : 8);
    hipLaunchKernelGGL((score_stream_lds_kernel<ST, kStats, kBf16>), dim3(grid), dim3(64), 0,
                       stream, a, n_items);
  }
}

// The tile (or streaming) kernel alone; returns the streaming choice.
template <bool kStats, bool kBf16>
static int launch_tiles_t(const ScoreArgs& a, hipStream_t stream) {
  const int st = stream_tokens(a.T);
  if (st == 1) launch_stream<1, kStats, kBf16>(a, stream);
  else if (st == 2) launch_stream<2, kStats, kBf16>(a, stream);
  else if (st == 4) launch_stream<4, kStats, kBf16>(a, stream);
  else {
    const unsigned grid = (unsigned)a.n_vt * (unsigned)a.n_tt;
    hipLaunchKernelGGL((score_tile_kernel<kStats, kBf16>), dim3(grid), dim3(kThreads), 0, stream,
                       a);
  }
  return st;
}

template <bool kStats>
static int launch_tiles(const ScoreArgs& a, hipStream_t stream) {
  return a.bf16_logits ? launch_tiles_t<kStats, true>(a, stream)
                       : launch_tiles_t<kStats, false>(a, stream);
}

template <bool kStats>
static hipError_t launch_score_t(const ScoreArgs& a, hipStream_t stream) {
  const int st = launch_tiles<kStats>(a, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (st)
    hipLaunchKernelGGL((lse_merge_kernel<true, kStats>), dim3((a.T + 63) / 64),
                       dim3(64 * kMergeSegs), 0, stream, a);
  else
    hipLaunchKernelGGL((lse_merge_kernel<false, kStats>), dim3((a.T + 63) / 64),
                       dim3(64 * kMergeSegs), 0, stream, a);
  return hipGetLastError();
}

template <bool kStats>
static hipError_t launch_shard_t(const ScoreArgs& a, const ShardArgs& s, hipStream_t stream) {
  // A shard with no rows (more shards than segments hold tiles) still writes
  // the empty records of its segments.
  const int st = a.n_vt > 0 ? launch_tiles<kStats>(a, stream) : stream_tokens(a.T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((a.T + 63) / 64), (unsigned)s.n_seg);
  if (st)
    hipLaunchKernelGGL((shard_fold_kernel<true, kStats>), grid, dim3(64), 0, stream, a, s);
  else
    hipLaunchKernelGGL((shard_fold_kernel<false, kStats>), grid, dim3(64), 0, stream, a, s);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t stream) {
  return a.out_ent ? launch_score_t<true>(a, stream) : launch_score_t<false>(a, stream);
}

int merge_segment_tiles(int64_t V_true) {
  const int64_t n_vt = (V_true + kTileV - 1) / kTileV;
  return (int)((n_vt + kMergeSegs - 1) / kMergeSegs);
}

hipError_t launch_score_shard(const ScoreArgs& a, const ShardArgs& s, hipStream_t stream) {
  return s.F == 5 ? launch_shard_t<true>(a, s, stream) : launch_shard_t<false>(a, s, stream);
}

hipError_t launch_merge_shards(const ScoreArgs& a, const ShardArgs& s, hipStream_t stream) {
  const dim3 grid((unsigned)((a.T + 255) / 256));
  if (s.F == 5) hipLaunchKernelGGL(shard_merge_kernel<true>, grid, dim3(256), 0, stream, a, s);
  else hipLaunchKernelGGL(shard_merge_kernel<false>, grid, dim3(256), 0, stream, a, s);
  return hipGetLastError();
}

}  // namespace lp
