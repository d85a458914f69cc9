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
//  * One workgroup = 4 waves computes a 256 (vocab) x 256 (token) tile of
//    Z^T = W . X^T with v_mfma_f32_32x32x16_bf16, fp32 accumulation, the whole
//    hidden dimension in ascending 64-wide LDS stages (no split-K). Each wave
//    owns 128 x 128 outputs = 4 x 4 MFMA tiles (256 accumulator registers).
//    Tokens are the MFMA "N" dimension, so every lane holds one token column
//    and 16 vocabulary rows per MFMA tile: the vocabulary reduction is mostly
//    inside a lane.
//  * Operand tiles are staged global -> registers -> LDS, double buffered,
//    one barrier per stage; 16-byte chunks are XOR-swizzled per row so that
//    the ds_read_b128 fragment reads do not collide on LDS banks.
//  * Epilogue: scale by log2(e)/temperature, mask rows >= V_true to -inf,
//    per-token max and sum of exp2 over the lane's 64 values, the lane pair
//    (l, l^32) and the two vocabulary waves, in a fixed order; write one
//    (max, sum) partial per (vocabulary tile, token); the single lane that
//    holds the target logit writes it. Logits never reach memory.
//  * A second kernel merges the vocabulary tiles of each token in ascending
//    tile order and writes logprob and log-sum-exp in nats.
//
// Batch invariance: the arithmetic applied to a (token, vocabulary row) pair
// depends only on the tile shape, H and the vocabulary tile index, never on
// T, on the token's slot in its tile, on the other tokens or on which CU runs
// the tile. Rows past T are clamped copies whose results are discarded.
#include <math.h>

#include "lp_internal.h"

namespace lp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaveV = 128;                  // vocab rows per wave
constexpr int kWaveT = 128;                  // token columns per wave
constexpr int kSubV = kWaveV / 32;           // MFMA tiles along vocab
constexpr int kSubT = kWaveT / 32;           // MFMA tiles along tokens
constexpr int kStageBytes = kTileV * kTileK * 2;     // one operand stage: 32 KiB
constexpr int kLoads = kStageBytes / 16 / kThreads;  // 16-byte copies per thread per operand
// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4],
// lgkmcnt [11:8]); only vmcnt is constrained.
constexpr int kWaitVm0 = 0x0F70;             // vmcnt(0)
constexpr int kGroupV = 4;                   // vocab tiles per scheduling group
constexpr float kLn2 = 0.693147180559945309f;

static_assert(kTileV == kTileT, "A and B stages share one layout");
static_assert(kTileV == 2 * kWaveV && kTileT == 2 * kWaveT, "2 x 2 waves");
static_assert(kLoads * kThreads * 16 == kStageBytes, "stage split");

// Physical 16-byte chunk of logical chunk `c` in tile row `row`.
__device__ __forceinline__ int swz(int row, int c) {
  return c ^ ((row ^ (row >> 3)) & 7);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }


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

// Enqueue copies j0 <= j < j1 of one K stage of both operands into the LDS
// stage buffers dstA (W) and dstB (X).
__device__ __forceinline__ void issue_stage(__amdgpu_buffer_rsrc_t wres, __amdgpu_buffer_rsrc_t xres,
                                            const uint32_t (&offA)[kLoads],
                                            const uint32_t (&offB)[kLoads], lds_char* dstA,
                                            lds_char* dstB, int wave, int koff, int j0, int j1) {
#pragma unroll
  for (int j = j0; j < j1; ++j) {
    const int q = 4 * j + wave;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void*)(dstA + q * 1024), 16, offA[j],
                                             koff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void*)(dstB + q * 1024), 16, offB[j],
                                             koff, 0, 0);
  }
}

// ---- Epilogue pieces shared by both tile kernels, so that a (token,
// vocabulary tile) pair goes through the same floating-point operations in the
// same order whichever kernel scores it. A wave holds kSubV MFMA tiles of 32
// vocabulary rows for each token column; `v(i, r)` returns the raw accumulator
// of vocabulary sub-tile i, register r, for the lane's token. MFMA 32x32
// output layout: lane l holds column (l & 31) and, in register r, row
// 8 * (r >> 2) + 4 * (l >> 5) + (r & 3).

// Per-token max and sum of exp2 over the wave's 128 rows (lane pair l, l^32).
// The scale log2(e)/T is positive, so the max of the scaled logits is the
// scaled max; the scale is folded into the exp2 argument with one FMA.
template <class Get>
__device__ __forceinline__ void wave_lse(Get v, float scale2, float& m_out, float& s_out) {
  const float NEG_INF = -__builtin_inff();
  float mr = NEG_INF;
#pragma unroll
  for (int i = 0; i < kSubV; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) mr = fmaxf(mr, v(i, r));
  mr = fmaxf(mr, __shfl_xor(mr, 32));
  const float m = mr * scale2;
  float s = 0.f;
  if (mr != NEG_INF) {
#pragma unroll
    for (int i = 0; i < kSubV; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += fast_exp2(__builtin_fmaf(v(i, r), scale2, -m));
  }
  s += __shfl_xor(s, 32);  // s_l + s_{l^32}: identical in both lanes
  m_out = m;
  s_out = s;
}

// Target gather for token t: exactly one lane of the grid holds (target, t);
// wv_lo is the first vocabulary row of the wave.
template <class Get>
__device__ __forceinline__ void gather_target(Get v, const ScoreArgs& a, int t, int64_t wv_lo,
                                              int fhalf) {
  const int64_t tgt = a.ids[t];
  const int64_t loc = tgt - wv_lo;
  if (tgt >= 0 && tgt < a.V_true && loc >= 0 && loc < kWaveV) {
    const int li = (int)loc;
    const int rr = li & 31;
    if (((rr >> 2) & 1) == fhalf) {
      // Flat (sub-tile, register) index of the target row; a branch-free
      // select over the lane's values picks it.
      const int k = (li >> 5) * 16 + (((rr >> 3) << 2) | (rr & 3));
      float tv = 0.f;
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) tv = (k == i * 16 + r) ? v(i, r) : tv;
      a.tval[t] = tv * a.scale2;
    }
  }
}

// Merge of the two 128-row halves of a vocabulary tile, lower half first
// (m0 is finite: row v0 < V_true lies in the lower half).
__device__ __forceinline__ void merge_halves(float m0, float s0, float m1, float s1, float& M,
                                             float& S) {
  M = fmaxf(m0, m1);
  S = __builtin_fmaf(s1, fast_exp2(m1 - M), s0 * fast_exp2(m0 - M));  // contraction spelled out
}

// Rows at or past V_true (only in the last vocabulary tile) read as -inf:
// register r of vocabulary sub-tile i holds row vlane + 32 i + 8 (r >> 2) +
// (r & 3), vlane = first vocabulary row of the wave + 4 (lane >> 5). The
// epilogue takes this masked view only in that tile (a uniform branch), so
// the accumulators are never rewritten.
#define LP_MASKED(x_, vlane_, i_, r_, V_) \
  (((vlane_) + 32 * (i_) + 8 * ((r_) >> 2) + ((r_) & 3) >= (V_)) ? -__builtin_inff() : (x_))

__global__ __launch_bounds__(kThreads, 1) void score_tile_kernel(ScoreArgs a) {
  // LDS: two stages of each operand, 256 rows x 128 B each, the 16-byte chunks
  // of row r XOR-permuted by f(r) (see swz()). Separate objects, so the
  // compiler can tell the copies into one stage from the reads of the other.
  __shared__ __attribute__((aligned(1024))) char sA0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kStageBytes];
  __shared__ float red_m[2][kTileT];
  __shared__ float red_s[2][kTileT];

  int vt, tt;
  tile_of(blockIdx.x, a.n_vt, a.n_tt, kGroupV, vt, tt);
  vt = __builtin_amdgcn_readfirstlane(vt);  // uniform: keep tile state in SGPRs
  tt = __builtin_amdgcn_readfirstlane(tt);
  const int v0 = vt * kTileV, t0 = tt * kTileT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  // ---- Global -> LDS assignment. Per operand and stage, wave w issues 8
  // copies; copy j fills LDS rows 8q .. 8q+7 (q = 4 j + w), lane i writing
  // physical chunk (i & 7) of row 8q + (i >> 3), i.e. logical chunk
  // (i & 7) ^ f(row). Rows past the matrix are clamped (results discarded).
  // Buffer resources based at the first row of each operand tile: the copies
  // then take a 32-bit per-lane offset plus a uniform K offset.
  const char* wtile = reinterpret_cast<const char*>(a.w) + (size_t)v0 * a.H * 2;
  const char* xtile = reinterpret_cast<const char*>(a.x) + (size_t)t0 * a.ldh * 2;
  const uint32_t w_span = span_bytes((uint64_t)(a.V_rows - v0) * (uint64_t)a.H * 2);
  const uint32_t x_span = span_bytes((uint64_t)(a.T - t0 - 1) * (uint64_t)a.ldh * 2 + (uint64_t)a.H * 2);
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(wtile, w_span);
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(xtile, x_span);
  uint32_t offA[kLoads], offB[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int q = 4 * j + wave;
    const int row = 8 * q + (lane >> 3);
    const int c = swz(row, lane & 7);  // XOR permutation is its own inverse
    const int ra = min(row, a.V_rows - 1 - v0);
    const int rt = min(row, a.T - 1 - t0);
    offA[j] = (uint32_t)ra * (uint32_t)(a.H * 2) + c * 16;
    offB[j] = (uint32_t)rt * (uint32_t)(a.ldh * 2) + c * 16;
  }
#define ISSUE_PART(kt_, buf_, j0_, j1_)                                                 \
  issue_stage(wres, xres, offA, offB, (lds_char*)((buf_) ? sA1 : sA0),               \
              (lds_char*)((buf_) ? sB1 : sB0), wave, (kt_) * (kTileK * 2), (j0_), (j1_))
#define ISSUE_STAGE(kt_, buf_) ISSUE_PART((kt_), (buf_), 0, kLoads)

  // ---- Fragment reads. Lane l reads row (base + 32 i + (l & 31)), logical
  // chunk 2 s + (l >> 5). With f(row) = (l & 7) ^ ((l & 31) >> 3) ^ 4 (i & 1)
  // the physical chunk is 2 (s ^ 2 (i & 1)) ^ c0 with c0 = (l >> 5) ^ f0, so
  // four addresses per operand cover every (s, i); the rest is immediate.
  const int frow = lane & 31, fhalf = lane >> 5;
  const int c0 = fhalf ^ ((frow & 7) ^ (frow >> 3));
  uint32_t rdA[4], rdB[4];
#pragma unroll
  for (int sp = 0; sp < 4; ++sp) {
    rdA[sp] = (uint32_t)((wm * kWaveV + frow) * 128 + (((2 * sp) ^ c0) * 16));
    rdB[sp] = (uint32_t)((wn * kWaveT + frow) * 128 + (((2 * sp) ^ c0) * 16));
  }
  auto read_frags = [&](bf16x8 (&fa)[kSubV], bf16x8 (&fb)[kSubT], int buf, int s)
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSubV; ++i) {
      const int sp = s ^ (2 * (i & 1));
      fa[i] = *reinterpret_cast<const bf16x8*>((buf ? sA1 : sA0) + rdA[sp] + i * 4096);
    }
#pragma unroll
    for (int j = 0; j < kSubT; ++j) {
      const int sp = s ^ (2 * (j & 1));
      fb[j] = *reinterpret_cast<const bf16x8*>((buf ? sB1 : sB0) + rdB[sp] + j * 4096);
    }
  };

  f32x16 acc[kSubV][kSubT];
#pragma unroll
  for (int i = 0; i < kSubV; ++i)
#pragma unroll
    for (int j = 0; j < kSubT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto mma = [&](const bf16x8 (&fa)[kSubV], const bf16x8 (&fb)[kSubT])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSubV; ++i)
#pragma unroll
      for (int j = 0; j < kSubT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  const int nk = a.H / kTileK;
  bf16x8 fa0[kSubV], fb0[kSubT], fa1[kSubV], fb1[kSubT];

  // Software pipeline over K stages. Phase kt runs between two barriers with
  // stage kt readable in LDS buffer kt & 1 and four substeps of 16 MFMAs. The
  // copies of stage kt+1 into the other buffer (freed by the barrier just
  // passed) are spread one per two MFMAs over the first two substeps: a
  // 1-KiB copy keeps the CU's address unit busy for several cycles, and
  // bursts of copies from the four waves (which all leave the barrier
  // together) would stall their in-order MFMA issue, while copies issued in
  // the second half of the phase would not land before its end. Fragment
  // registers alternate per substep so that the LDS reads of substep s+1
  // (one per two MFMAs) overlap the MFMAs of substep s; the 16 MFMAs of the
  // last substep are carried into the next phase, where they cover the
  // latency of its first reads. Each phase ends with vmcnt(0) + barrier, so
  // no copy is in flight across the loop back-edge. The copy of the next
  // stage is issued unconditionally (branch-free, so it can be interleaved):
  // in the last phase it re-copies the final stage into the idle buffer,
  // which nothing reads. sched_barrier(0) keeps the compiler from re-ordering
  // the substeps; sched_group_barrier sets the interleave inside one (masks:
  // 0x008 MFMA, 0x020 VMEM read, 0x100 DS read).
#define PHASE_FENCE() __builtin_amdgcn_sched_barrier(0)
#define SGB(mask_, n_) __builtin_amdgcn_sched_group_barrier((mask_), (n_), 0)
#define MIX_READS()                                  \
  do {                                               \
    _Pragma("unroll") for (int u = 0; u < 8; ++u) {  \
      SGB(0x008, 1);                                 \
      SGB(0x100, 1);                                 \
      SGB(0x008, 1);                                 \
    }                                                \
  } while (0)
#define MIX_READS_COPIES()                           \
  do {                                               \
    _Pragma("unroll") for (int u = 0; u < 8; ++u) {  \
      SGB(0x008, 1);                                 \
      SGB(0x020, 1);                                 \
      SGB(0x100, 1);                                 \
      SGB(0x008, 1);                                 \
    }                                                \
  } while (0)
#define PHASE(kt_, buf_, carry_)                                            \
  do {                                                                      \
    const int buf = (buf_);                                                 \
    const int kc = min((kt_) + 1, nk - 1);                                  \
    ISSUE_PART(kc, buf ^ 1, 0, kLoads / 2);                                 \
    read_frags(fa0, fb0, buf, 0);                                           \
    if (carry_) {                                                           \
      mma(fa1, fb1);                                                        \
      MIX_READS_COPIES();                                                   \
    }                                                                       \
    PHASE_FENCE();                                                          \
    ISSUE_PART(kc, buf ^ 1, kLoads / 2, kLoads);                            \
    read_frags(fa1, fb1, buf, 1);                                           \
    mma(fa0, fb0);                                                          \
    MIX_READS_COPIES();                                                     \
    PHASE_FENCE();                                                          \
    read_frags(fa0, fb0, buf, 2);                                           \
    mma(fa1, fb1);                                                          \
    MIX_READS();                                                            \
    PHASE_FENCE();                                                          \
    read_frags(fa1, fb1, buf, 3);                                           \
    mma(fa0, fb0);                                                          \
    MIX_READS();                                                            \
    PHASE_FENCE();                                                          \
    __builtin_amdgcn_s_waitcnt(kWaitVm0);                                   \
    __syncthreads();                                                        \
    PHASE_FENCE();                                                          \
  } while (0)

  ISSUE_STAGE(0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  PHASE(0, 0, false);
  for (int kt = 1; kt < nk; kt += 2) {
    PHASE(kt, 1, true);
    if (kt + 1 < nk) PHASE(kt + 1, 0, true);
  }
  mma(fa1, fb1);  // last substep of the last stage
#undef ISSUE_STAGE
#undef ISSUE_PART
#undef PHASE
#undef MIX_READS
#undef MIX_READS_COPIES
#undef SGB
#undef PHASE_FENCE

  // ---- Epilogue: per-token online LSE over this wave's 128 vocab rows. ----
  const int vlane = v0 + wm * kWaveV + 4 * fhalf;
  const bool vtail = v0 + kTileV > a.V_true;
  const int64_t wv_lo = v0 + wm * kWaveV;

#pragma unroll
  for (int j = 0; j < kSubT; ++j) {
    const int tl = wn * kWaveT + j * 32 + frow;
    const int t = t0 + tl;
    auto v = [&](int i, int r) __attribute__((always_inline)) { return acc[i][j][r]; };
    auto vm = [&](int i, int r) __attribute__((always_inline)) {
      return LP_MASKED(acc[i][j][r], vlane, i, r, a.V_true);
    };
    float m, s;
    if (vtail) wave_lse(vm, a.scale2, m, s);
    else wave_lse(v, a.scale2, m, s);
    if (t < a.T) gather_target(v, a, t, wv_lo, fhalf);  // targets lie below V_true
    if (fhalf == 0) {
      red_m[wm][tl] = m;
      red_s[wm][tl] = s;
    }
  }
  __syncthreads();

  {
    const int tl = tid;
    const int t = t0 + tl;
    float M, S;
    merge_halves(red_m[0][tl], red_s[0][tl], red_m[1][tl], red_s[1][tl], M, S);
    if (t < a.T) {
      a.part_m[(size_t)vt * a.T + t] = M;
      a.part_s[(size_t)vt * a.T + t] = S;
    }
  }
}

// ---- Streaming kernel for small batches (HBM-bound on W). ----
// With few rows the product is a stream over W (2 V H bytes) and the 256 x 256
// tiles would be mostly padding. Here a work item is one 128-row half of a
// vocabulary tile x 32 ST tokens, computed by a single wave in exactly the
// placement of the 256 x 256 kernel -- vocabulary row -> (MFMA tile i, lane
// half, register), token -> MFMA column, the same v_mfma_f32_32x32x16_bf16
// chain over 16-wide K blocks in ascending order -- and the same per-wave
// epilogue (wave_lse), so every row's bits match. The wave writes its half's
// (max, sum) partial; the merge kernel applies merge_halves before folding
// the tiles, as the 256 x 256 kernel does in LDS.
//
// The grid is persistent (a fixed number of one-wave workgroups per CU, each
// taking items b, b + G, b + 2G, ... with XCD-contiguous numbering, token
// tiles fastest so the waves of one XCD that share a W half-tile run
// together). Each wave streams its items' 64-wide K stages (128-byte row
// segments of W) through a ring of kSmStages LDS slots with direct buffer ->
// LDS copies, kSmStages - 1 stages in flight, continuing across item
// boundaries; being alone in its workgroup, a wave only waits on its own
// vmcnt, never on a barrier. Two slots (four waves per CU) stream faster than
// deeper rings with fewer waves per CU.
constexpr int kSmK = 64;                       // hidden elements per stage
constexpr int kSmStages = 2;                   // ring depth
constexpr int kSmRowB = kSmK * 2;              // LDS row bytes
constexpr int kSmNC = kSmRowB / 16;            // 16-byte chunks per row
constexpr int kSmRPC = 1024 / kSmRowB;         // rows per 1-KiB wave copy
constexpr int kSmRowsA = kWaveV;               // 128 W rows per item
constexpr int kSmCopiesA = kSmRowsA * kSmRowB / 1024;
static_assert(kSmNC == 4 || kSmNC == 8, "64- or 128-byte rows");

// Physical chunk of logical chunk c in row `row`: conflict-free fragment
// reads for 64-byte rows ((row >> 2) & 3) and 128-byte rows (as in the
// 256 x 256 kernel).
__host__ __device__ __forceinline__ int swz_sm(int row, int c) {
  return kSmNC == 4 ? c ^ ((row >> 2) & 3) : c ^ ((row ^ (row >> 3)) & 7);
}

template <int ST>
struct Stream {
  static constexpr int kTok = 32 * ST;                     // tokens per item
  static constexpr int kCopiesB = kTok * kSmRowB / 1024;   // 2 ST
  static constexpr int kCopies = kSmCopiesA + kCopiesB;    // per stage
  static constexpr int kSlotA = kSmRowsA * kSmRowB;        // 8 KiB
  static constexpr int kSlotB = kTok * kSmRowB;            // 2 ST KiB
  static constexpr int kSlot = kSlotA + kSlotB;
  static constexpr int kLds = kSmStages * kSlot;
  static_assert((kSmStages - 1) * kCopies <= 63, "vmcnt holds at most 63");
};

template <int ST>
__global__ __launch_bounds__(64) void score_stream_kernel(ScoreArgs a, int n_items) {
  using S = Stream<ST>;
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
  // logical chunk swz_sm(row, i % kSmNC) (the permutation is an involution).
  const int lrow = lane / kSmNC;
#define SM_LC(q_) ((uint32_t)(swz_sm(kSmRPC * (q_) + lrow, lane % kSmNC) * 16))

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
    lds_char* slot = (lds_char*)ring + (g % kSmStages) * S::kSlot;
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

  // Fragment reads: row 32 i + (l & 31) of the half-tile (A) or 32 j + (l & 31)
  // of the token tile (B), logical chunk 2 s + (l >> 5).
  const int frow = lane & 31, fhalf = lane >> 5;
#define SM_RD(row0_, sp_) \
  ((uint32_t)(((row0_) + frow) * kSmRowB + swz_sm((row0_) + frow, 2 * (sp_) + fhalf) * 16))

  f32x16 acc[kSubV][ST];
  for (int g = 0; g < kSmStages - 1 && g < n_stages; ++g) issue(g);
  for (int g = 0; g < n_stages; ++g) {
    if (g + kSmStages - 1 < n_stages) {
      issue(g + kSmStages - 1);
      // Stage g has landed once at most (kSmStages - 1) stages' copies remain.
      __builtin_amdgcn_s_waitcnt(0x0F70 | (((kSmStages - 1) * S::kCopies) & 15) |
                                 ((((kSmStages - 1) * S::kCopies) >> 4) << 14));
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    const int kt = g % nk;
    if (kt == 0) {
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
#pragma unroll
        for (int jj = 0; jj < ST; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;
    }
    const char* slot = ring + (g % kSmStages) * S::kSlot;
#pragma unroll
    for (int sp = 0; sp < kSmK / 16; ++sp) {
      bf16x8 fa[kSubV], fb[ST];
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(slot + SM_RD(32 * i, sp));
#pragma unroll
      for (int jj = 0; jj < ST; ++jj)
        fb[jj] = *reinterpret_cast<const bf16x8*>(slot + S::kSlotA + SM_RD(32 * jj, sp));
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
#pragma unroll
        for (int jj = 0; jj < ST; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[jj], acc[i][jj], 0, 0, 0);
    }
    if (kt == nk - 1) {
      const int L = xb + (g / nk) * G;
      const int vh = L / a.n_tt, tt = L - vh * a.n_tt;
      const int vbase = vh * kWaveV, t0 = tt * S::kTok;
      const int vlane = vbase + 4 * fhalf;
      const bool vtail = vbase + kWaveV > a.V_true;
#pragma unroll
      for (int jj = 0; jj < ST; ++jj) {
        const int t = t0 + 32 * jj + frow;
        auto v = [&](int i, int r) __attribute__((always_inline)) { return acc[i][jj][r]; };
        auto vm = [&](int i, int r) __attribute__((always_inline)) {
          return LP_MASKED(acc[i][jj][r], vlane, i, r, a.V_true);
        };
        float m, s;
        if (vtail) wave_lse(vm, a.scale2, m, s);
        else wave_lse(v, a.scale2, m, s);
        if (t < a.T) {
          gather_target(v, a, t, vbase, fhalf);  // targets lie below V_true
          if (fhalf == 0) {
            a.part_m[(size_t)vh * a.T + t] = m;
            a.part_s[(size_t)vh * a.T + t] = s;
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
constexpr int kMergeSegs = 16;

__device__ __forceinline__ void lse_fold(float& M, float& S, float m, float s) {
  const float Mn = fmaxf(M, m);
  // exp2(-inf) = 0 on first use; the contraction is spelled out.
  S = __builtin_fmaf(s, fast_exp2(m - Mn), S * fast_exp2(M - Mn));
  M = Mn;
}

// kHalves: the partials are per 128-row half of each vocabulary tile (rows
// 2 vt and 2 vt + 1), merged with merge_halves first.
template <bool kHalves>
__global__ __launch_bounds__(64 * kMergeSegs) void lse_merge_kernel(ScoreArgs a) {
  __shared__ float seg_m[kMergeSegs][64];
  __shared__ float seg_s[kMergeSegs][64];
  const int lane = threadIdx.x & 63, seg = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + lane;
  const int per = (a.n_vt + kMergeSegs - 1) / kMergeSegs;
  const int lo = min(a.n_vt, seg * per), hi = min(a.n_vt, lo + per);
  float M = -__builtin_inff(), S = 0.f;
  if (t < a.T) {
    const float* pm = a.part_m + t;
    const float* ps = a.part_s + t;
    if (kHalves) {
#pragma unroll 8
      for (int vt = lo; vt < hi; ++vt) {
        float m, s;
        merge_halves(pm[(size_t)(2 * vt) * a.T], ps[(size_t)(2 * vt) * a.T],
                     pm[(size_t)(2 * vt + 1) * a.T], ps[(size_t)(2 * vt + 1) * a.T], m, s);
        lse_fold(M, S, m, s);
      }
    } else {
#pragma unroll 8
      for (int vt = lo; vt < hi; ++vt)
        lse_fold(M, S, pm[(size_t)vt * a.T], ps[(size_t)vt * a.T]);
    }
  }
  seg_m[seg][lane] = M;
  seg_s[seg][lane] = S;
  __syncthreads();
  if (seg != 0 || t >= a.T) return;
  M = seg_m[0][lane];
  S = seg_s[0][lane];
#pragma unroll
  for (int g = 1; g < kMergeSegs; ++g)  // an empty segment (-inf, 0) folds to a no-op
    lse_fold(M, S, seg_m[g][lane], seg_s[g][lane]);
  const float lse2 = M + fast_log2(S);
  const int64_t id = a.ids[t];
  const bool ok = id >= 0 && id < a.V_true;
  a.out_lp[t] = ok ? (a.tval[t] - lse2) * kLn2 : __builtin_nanf("");
  if (a.out_lse) a.out_lse[t] = lse2 * kLn2;
  if (!ok && a.bad_rows) atomicAdd(a.bad_rows, 1);
}

}  // namespace

// Streaming kernel choice: items of 32 ST tokens; 0 = the 256 x 256 kernel.
static int stream_tokens(int64_t T) {
  if (T <= 32) return 1;
  if (T <= kSkinnyMaxT) return 2;
  return 0;
}

ScoreWorkspace score_workspace_layout(int64_t T, int64_t V_true) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t n_vt = (size_t)((V_true + kTileV - 1) / kTileV);
  const size_t rows = stream_tokens(T) ? 2 * n_vt : n_vt;  // half-tile partials
  ScoreWorkspace w;
  w.off_m = 0;
  w.off_s = up(w.off_m + rows * (size_t)T * sizeof(float));
  w.off_t = up(w.off_s + rows * (size_t)T * sizeof(float));
  w.total = up(w.off_t + (size_t)T * sizeof(float));
  return w;
}

template <int ST>
static void launch_stream(ScoreArgs a, hipStream_t stream) {
  a.n_tt = (a.T + 32 * ST - 1) / (32 * ST);
  const int n_items = 2 * a.n_vt * a.n_tt;
  // Workgroups (one wave each) per CU: as many as the LDS ring allows.
  const int per_cu = (160 * 1024) / Stream<ST>::kLds;
  const int grid = 256 * (per_cu < 8 ? per_cu : 8);
  hipLaunchKernelGGL(score_stream_kernel<ST>, dim3(grid), dim3(64), 0, stream, a, n_items);
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t stream) {
  const int st = stream_tokens(a.T);
  if (st == 1) launch_stream<1>(a, stream);
  else if (st == 2) launch_stream<2>(a, stream);
  else {
    const unsigned grid = (unsigned)a.n_vt * (unsigned)a.n_tt;
    hipLaunchKernelGGL(score_tile_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (st)
    hipLaunchKernelGGL(lse_merge_kernel<true>, dim3((a.T + 63) / 64), dim3(64 * kMergeSegs), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(lse_merge_kernel<false>, dim3((a.T + 63) / 64), dim3(64 * kMergeSegs), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace lp
