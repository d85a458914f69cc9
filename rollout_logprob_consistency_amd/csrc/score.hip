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
constexpr int kChunks = kTileK / 8;          // 16-byte chunks per row per stage
constexpr int kStageU4 = kTileV * kChunks;   // uint4 per operand stage
constexpr int kLoads = kStageU4 / kThreads;  // 16-byte loads per thread per operand
constexpr int kGroupV = 4;                   // vocab tiles per scheduling group
constexpr float kLn2 = 0.693147180559945309f;

static_assert(kTileV == kTileT, "A and B stages share one layout");
static_assert(kTileV == 2 * kWaveV && kTileT == 2 * kWaveT, "2 x 2 waves");
static_assert(kLoads * kThreads == kStageU4, "stage split");

// Physical 16-byte chunk of logical chunk `c` in tile row `row`.
__device__ __forceinline__ int swz(int row, int c) {
  return c ^ ((row ^ (row >> 3)) & 7);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Workgroup id -> (vocab tile, token tile). The hardware deals workgroups to
// the 8 XCDs round-robin; give each XCD a contiguous run of logical tiles, and
// order logical tiles in groups of kGroupV vocab tiles with the token tile
// varying fastest, so the workgroups resident on one XCD share W and X slabs
// in that XCD's L2.
__device__ __forceinline__ void tile_of(int b, int n_vt, int n_tt, int& vt, int& tt) {
  const int G = n_vt * n_tt;
  const int xcd = b & 7, idx = b >> 3;
  const int per = G >> 3, rem = G & 7;
  const int L = (xcd < rem) ? xcd * (per + 1) + idx
                            : rem * (per + 1) + (xcd - rem) * per + idx;
  const int group = kGroupV * n_tt;
  const int g = L / group;
  const int first = g * kGroupV;
  const int gv = min(kGroupV, n_vt - first);
  const int r = L - g * group;
  vt = first + r % gv;
  tt = r / gv;
}

__global__ __launch_bounds__(kThreads, 1) void score_tile_kernel(ScoreArgs a) {
  __shared__ uint4 smem[4 * kStageU4];  // A0 | A1 | B0 | B1  (128 KiB)
  __shared__ float red_m[2][kTileT];
  __shared__ float red_s[2][kTileT];

  int vt, tt;
  tile_of(blockIdx.x, a.n_vt, a.n_tt, vt, tt);
  const int v0 = vt * kTileV, t0 = tt * kTileT;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // Global -> LDS assignment: 16-byte chunk (row, kc) with row = lrow + 32 j.
  const int lrow = tid >> 3, kc = tid & 7;
  const uint16_t* pa[kLoads];
  const uint16_t* pb[kLoads];
  int woff[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int row = lrow + 32 * j;
    const int rv = min(v0 + row, a.V_rows - 1);
    const int rt = min(t0 + row, a.T - 1);
    pa[j] = a.w + (size_t)rv * a.H + kc * 8;
    pb[j] = a.x + (size_t)rt * a.ldh + kc * 8;
    woff[j] = row * kChunks + swz(row, kc);
  }

  uint4 ra[kLoads], rb[kLoads];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      ra[j] = *reinterpret_cast<const uint4*>(pa[j] + kt * kTileK);
      rb[j] = *reinterpret_cast<const uint4*>(pb[j] + kt * kTileK);
    }
  };
  auto swrite = [&](int buf) {
    uint4* As = smem + buf * kStageU4;
    uint4* Bs = smem + (2 + buf) * kStageU4;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      As[woff[j]] = ra[j];
      Bs[woff[j]] = rb[j];
    }
  };

  // Fragment read offsets (uint4 units within a stage) for substep s, tile i.
  const int frow = lane & 31, fhalf = lane >> 5;

  f32x16 acc[kSubV][kSubT];
#pragma unroll
  for (int i = 0; i < kSubV; ++i)
#pragma unroll
    for (int j = 0; j < kSubT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = a.H / kTileK;
  gload(0);
  swrite(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint4* As = smem + cur * kStageU4;
    const uint4* Bs = smem + (2 + cur) * kStageU4;
#pragma unroll
    for (int s = 0; s < kTileK / 16; ++s) {
      const int ch = 2 * s + fhalf;
      bf16x8 fa[kSubV], fb[kSubT];
#pragma unroll
      for (int i = 0; i < kSubV; ++i) {
        const int row = wm * kWaveV + i * 32 + frow;
        fa[i] = as_bf16x8(As[row * kChunks + swz(row, ch)]);
      }
#pragma unroll
      for (int j = 0; j < kSubT; ++j) {
        const int row = wn * kWaveT + j * 32 + frow;
        fb[j] = as_bf16x8(Bs[row * kChunks + swz(row, ch)]);
      }
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
#pragma unroll
        for (int j = 0; j < kSubT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) swrite(cur ^ 1);
    __syncthreads();
  }

  // ---- Epilogue: per-token online LSE over this wave's 128 vocab rows. ----
  // MFMA 32x32 output layout: lane l holds column (l & 31) and, in register
  // r, row 8 * (r >> 2) + 4 * (l >> 5) + (r & 3).
  const float NEG_INF = -__builtin_inff();
  const int vlane = v0 + wm * kWaveV + 4 * fhalf;  // + 32 i + 8 (r >> 2) + (r & 3)
  const bool vtail = v0 + kTileV > a.V_true;
  const int64_t wv_lo = v0 + wm * kWaveV;

#pragma unroll
  for (int j = 0; j < kSubT; ++j) {
    const int tl = wn * kWaveT + j * 32 + frow;
    const int t = t0 + tl;
    float m = NEG_INF;
#pragma unroll
    for (int i = 0; i < kSubV; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = acc[i][j][r] * a.scale2;
        if (vtail && vlane + 32 * i + 8 * (r >> 2) + (r & 3) >= a.V_true) x = NEG_INF;
        acc[i][j][r] = x;
        m = fmaxf(m, x);
      }
    m = fmaxf(m, __shfl_xor(m, 32));
    float s = 0.f;
    if (m != NEG_INF) {
#pragma unroll
      for (int i = 0; i < kSubV; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += fast_exp2(acc[i][j][r] - m);
    }
    s += __shfl_xor(s, 32);  // s_l + s_{l^32}: identical in both lanes

    // Target gather: exactly one lane of the grid holds (target, t).
    if (t < a.T) {
      const int64_t tgt = a.ids[t];
      const int64_t loc = tgt - wv_lo;
      if (tgt >= 0 && tgt < a.V_true && loc >= 0 && loc < kWaveV) {
        const int li = (int)loc;
        const int ti = li >> 5, rr = li & 31;
        if (((rr >> 2) & 1) == fhalf) {
          const int tr = ((rr >> 3) << 2) | (rr & 3);
          float tv = 0.f;
#pragma unroll
          for (int i = 0; i < kSubV; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (i == ti && r == tr) tv = acc[i][j][r];
          a.tval[t] = tv;
        }
      }
    }
    if (fhalf == 0) {
      red_m[wm][tl] = m;
      red_s[wm][tl] = s;
    }
  }
  __syncthreads();

  // Merge the two vocabulary halves of the tile (lower half first).
  {
    const int tl = tid;
    const int t = t0 + tl;
    const float m0 = red_m[0][tl], m1 = red_m[1][tl];
    const float s0 = red_s[0][tl], s1 = red_s[1][tl];
    const float M = fmaxf(m0, m1);  // m0 is finite: row v0 < V_true is in half 0
    const float S = s0 * fast_exp2(m0 - M) + s1 * fast_exp2(m1 - M);
    if (t < a.T) {
      a.part_m[(size_t)vt * a.T + t] = M;
      a.part_s[(size_t)vt * a.T + t] = S;
    }
  }
}

// One thread per token: merge the vocabulary-tile partials in ascending tile
// order, then logprob = (target - lse) in nats.
__global__ __launch_bounds__(256) void lse_merge_kernel(ScoreArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  float M = -__builtin_inff(), S = 0.f;
  for (int vt = 0; vt < a.n_vt; ++vt) {
    const float m = a.part_m[(size_t)vt * a.T + t];
    const float s = a.part_s[(size_t)vt * a.T + t];
    const float Mn = fmaxf(M, m);
    S = S * fast_exp2(M - Mn) + s * fast_exp2(m - Mn);
    M = Mn;
  }
  const float lse2 = M + fast_log2(S);
  const int64_t id = a.ids[t];
  const bool ok = id >= 0 && id < a.V_true;
  a.out_lp[t] = ok ? (a.tval[t] - lse2) * kLn2 : __builtin_nanf("");
  if (a.out_lse) a.out_lse[t] = lse2 * kLn2;
  if (!ok && a.bad_rows) atomicAdd(a.bad_rows, 1);
}

}  // namespace

ScoreWorkspace score_workspace_layout(int64_t T, int64_t V_true) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t n_vt = (size_t)((V_true + kTileV - 1) / kTileV);
  ScoreWorkspace w;
  w.off_m = 0;
  w.off_s = up(w.off_m + n_vt * (size_t)T * sizeof(float));
  w.off_t = up(w.off_s + n_vt * (size_t)T * sizeof(float));
  w.total = up(w.off_t + (size_t)T * sizeof(float));
  return w;
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.n_vt * (unsigned)a.n_tt;
  hipLaunchKernelGGL(score_tile_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((a.T + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lp
