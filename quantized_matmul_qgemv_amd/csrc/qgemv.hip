// Decode GEMV over group-quantized weights (BaseRT, native-Metal LLM
// inference on Apple Silicon, §3.3: one GEMV kernel per quantization
// format, dequantization folded into the inner loop).
//
// y[n] = sum_g ( s[n,g] * sum_{k in g} q[n,k] x[k]  +  b[n,g] * sum_{k in g} x[k] )
//
// The kernel is HBM-bound: every packed weight byte is read exactly once.
// Work decomposition (one workgroup = 4 wave64s):
//   * a "unit" is one 64-code group of one row: GROUP_BYTES (16/32/64 B
//     for 2/4/8 bits) of codes plus one fp16 scale and one fp16 bias;
//   * LPR consecutive lanes share a row; lane lr takes the row's groups
//     lr, lr + LPR, lr + 2*LPR, ...  so one wave-wide 128-bit load covers
//     64/LPR rows with contiguous, fully used 16-byte pieces;
//   * each lane keeps UR rows in flight (independent accumulators) and the
//     next group's loads are issued before the current group is consumed;
//   * for small n, WK waves of a workgroup split a row's groups and meet in
//     LDS (deterministic, no atomics).
// Activations are staged once per workgroup in LDS in "paired" order (the
// order the register unpack produces codes in, see qmm_device.h), together
// with two per-group constants:
//     C[g] = sum_{k in g} magic(k) * x[k]       X[g] = sum_{k in g} x[k]
// so that   sum_k q_k x_k = dot(magic + q, x) - C[g]   needs no per-code
// subtraction: each packed word costs one shift, a few AND-ORs and one
// v_dot2_f32_f16 per two codes.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = 4;
constexpr int kXStride = 144;  // bytes per group of paired x in LDS (128 + 16 pad)

template <int BITS, int LPR, int UR, int WK>
struct GemvCfg {
  static constexpr int WR = kGemvWaves / WK;   // waves along rows
  static constexpr int RPW = 64 / LPR;         // rows per wave per pass
  static constexpr int ROWS = WR * UR * RPW;   // rows per workgroup
};

// Stage x[0 .. 64*groups) into LDS: paired halves plus (C[g], X[g]).
template <int BITS>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int groups,
                                        unsigned char* xp, float2* cx) {
  using F = Fmt<BITS>;
  constexpr int C = F::CODES_PER_WORD;
  constexpr int PPW = F::PAIRS_PER_WORD;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)g * 64);
    uint32_t d[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = src[i];
      d[4 * i + 0] = v.x; d[4 * i + 1] = v.y; d[4 * i + 2] = v.z; d[4 * i + 3] = v.w;
    }
    uint32_t out[32];
    float csum = 0.0f, xsum = 0.0f;
#pragma unroll
    for (int wd = 0; wd < F::WORDS_PER_GROUP; ++wd) {
#pragma unroll
      for (int p = 0; p < PPW; ++p) {
        const int klo = wd * C + pair_lo<BITS>(p);
        const int khi = wd * C + pair_hi<BITS>(p);
        const uint32_t lo = (d[klo >> 1] >> (16 * (klo & 1))) & 0xFFFFu;
        const uint32_t hi = (d[khi >> 1] >> (16 * (khi & 1))) & 0xFFFFu;
        out[wd * PPW + p] = lo | (hi << 16);
        const float xl = f16_bits_to_f32((uint16_t)lo);
        const float xh = f16_bits_to_f32((uint16_t)hi);
        csum += magic_value<BITS>(p) * xl;
        csum += magic_value<BITS>(p) * xh;
        xsum += xl;
        xsum += xh;
      }
    }
    u32x4* dst = reinterpret_cast<u32x4*>(xp + (size_t)g * kXStride);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dst[i] = u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
    cx[g] = make_float2(csum, xsum);
  }
}

template <int BITS, int LPR, int UR, int WK>
__device__ __forceinline__ void gemv_block(const GemvProblem& P, int row0, unsigned char* smem) {
  using F = Fmt<BITS>;
  using Cfg = GemvCfg<BITS, LPR, UR, WK>;
  constexpr int V4 = F::VEC4_PER_GROUP;
  constexpr int WPG = F::WORDS_PER_GROUP;
  constexpr int PPW = F::PAIRS_PER_WORD;

  const int groups = P.k >> 6;
  unsigned char* xp = smem;
  float2* cx = reinterpret_cast<float2*>(smem + (size_t)groups * kXStride);
  float* red = reinterpret_cast<float*>(cx + groups);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave / WK;
  const int wk = wave % WK;
  const int slot = lane / LPR;
  const int lr = lane % LPR;
  const int T = groups / LPR;

  int rows[UR];
  const uint32_t* wrow[UR];
  const uint16_t* srow[UR];
  const uint16_t* brow[UR];
#pragma unroll
  for (int u = 0; u < UR; ++u) {
    const int r = row0 + (wr * UR + u) * Cfg::RPW + slot;
    rows[u] = r;
    const size_t rc = (size_t)(r < P.n ? r : P.n - 1);
    wrow[u] = P.w + rc * (size_t)groups * WPG;
    srow[u] = P.s + rc * (size_t)groups;
    brow[u] = P.b + rc * (size_t)groups;
  }

  u32x4 wv[UR][V4];
  uint16_t sv[UR], bv[UR];
  auto issue = [&](int t) {
    const int g = t * LPR + lr;
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      if constexpr (BITS == 2) {
        // a 2-bit group is 16 bytes: one load
        wv[u][0] = *reinterpret_cast<const u32x4*>(wrow[u] + (size_t)g * WPG);
      } else {
#pragma unroll
        for (int v = 0; v < V4; ++v)
          wv[u][v] = reinterpret_cast<const u32x4*>(wrow[u] + (size_t)g * WPG)[v];
      }
      sv[u] = srow[u][g];
      bv[u] = brow[u][g];
    }
  };

  int t = wk;
  if (t < T) issue(t);
  stage_x<BITS>(P.x, groups, xp, cx);
  __syncthreads();

  float acc[UR];
#pragma unroll
  for (int u = 0; u < UR; ++u) acc[u] = 0.0f;

  for (; t < T; t += WK) {
    u32x4 cw[UR][V4];
    uint16_t cs[UR], cb[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) {
#pragma unroll
      for (int v = 0; v < V4; ++v) cw[u][v] = wv[u][v];
      cs[u] = sv[u];
      cb[u] = bv[u];
    }
    const int g = t * LPR + lr;
    if (t + WK < T) issue(t + WK);

    uint32_t xr[32];
    const u32x4* xpv = reinterpret_cast<const u32x4*>(xp + (size_t)g * kXStride);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = xpv[i];
      xr[4 * i] = v.x; xr[4 * i + 1] = v.y; xr[4 * i + 2] = v.z; xr[4 * i + 3] = v.w;
    }
    const float2 c = cx[g];

#pragma unroll
    for (int u = 0; u < UR; ++u) {
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int j = 0; j < WPG; ++j) {
        const u32x4 v = cw[u][j >> 2];
        const uint32_t word = (j & 3) == 0 ? v.x : (j & 3) == 1 ? v.y : (j & 3) == 2 ? v.z : v.w;
        uint32_t h[PPW];
        unpack_word<BITS>(word, h);
#pragma unroll
        for (int p = 0; p < PPW; ++p) {
          if ((p & 1) == 0) a0 = dot2(h[p], xr[j * PPW + p], a0);
          else              a1 = dot2(h[p], xr[j * PPW + p], a1);
        }
      }
      const float s = f16_bits_to_f32(cs[u]);
      const float b = f16_bits_to_f32(cb[u]);
      acc[u] = fmaf(s, (a0 + a1) - c.x, fmaf(b, c.y, acc[u]));
    }
  }

#pragma unroll
  for (int u = 0; u < UR; ++u) {
    float v = acc[u];
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    acc[u] = v;
  }

  if constexpr (WK == 1) {
    if (lr == 0) {
#pragma unroll
      for (int u = 0; u < UR; ++u)
        if (rows[u] < P.n) P.y[rows[u]] = acc[u];
    }
  } else {
    if (lr == 0) {
#pragma unroll
      for (int u = 0; u < UR; ++u)
        red[((wr * UR + u) * Cfg::RPW + slot) * WK + wk] = acc[u];
    }
    __syncthreads();
    if (wk == 0 && lr == 0) {
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const float* r = red + ((wr * UR + u) * Cfg::RPW + slot) * WK;
        float v = r[0];
#pragma unroll
        for (int i = 1; i < WK; ++i) v += r[i];
        if (rows[u] < P.n) P.y[rows[u]] = v;
      }
    }
  }
}

template <int BITS, int LPR, int UR, int WK>
__global__ __launch_bounds__(kGemvThreads) void qgemv_kernel(GemvProblem P) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  gemv_block<BITS, LPR, UR, WK>(P, blockIdx.x * GemvCfg<BITS, LPR, UR, WK>::ROWS, smem);
}

template <int BITS, int LPR>
__global__ __launch_bounds__(kGemvThreads) void qgemv_batched_kernel(const GemvBlock* __restrict__ blocks) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const GemvBlock blk = blocks[blockIdx.x];
  gemv_block<BITS, LPR, 4, 1>(blk.p, blk.row0, smem);
}

// ------------------------------------------------------------------ host --

int gemv_rows_per_block(int lpr, int ur, int wk) { return (kGemvWaves / wk) * ur * (64 / lpr); }

int gemv_lanes_for_groups(int groups) {
  int lpr = 16;
  while (lpr > 1 && groups % lpr != 0) lpr >>= 1;
  return lpr;
}

GemvGeom gemv_choose(int n, int k) {
  const int groups = k / 64;
  GemvGeom g;
  g.lanes_per_row = gemv_lanes_for_groups(groups);
  const int T = groups / g.lanes_per_row;
  const int target = 1024;  // workgroups wanted to fill 256 CUs several times over
  g.row_unroll = 4;
  g.wave_ksplit = 1;
  auto blocks = [&](int ur, int wk) {
    const int r = gemv_rows_per_block(g.lanes_per_row, ur, wk);
    return (n + r - 1) / r;
  };
  if (blocks(4, 1) < target) g.row_unroll = 1;
  if (blocks(g.row_unroll, 1) < target && T >= 4) g.wave_ksplit = 4;
  g.rows_per_block = gemv_rows_per_block(g.lanes_per_row, g.row_unroll, g.wave_ksplit);
  return g;
}

size_t gemv_lds_bytes(int max_groups, const GemvGeom& g) {
  size_t bytes = (size_t)max_groups * (kXStride + sizeof(float2));
  if (g.wave_ksplit > 1) bytes += (size_t)g.rows_per_block * g.wave_ksplit * sizeof(float);
  return bytes;
}

template <int BITS, int LPR, int UR, int WK>
static hipError_t launch_one(const GemvProblem& p, hipStream_t st, size_t lds) {
  constexpr int ROWS = GemvCfg<BITS, LPR, UR, WK>::ROWS;
  const unsigned grid = (unsigned)((p.n + ROWS - 1) / ROWS);
  hipLaunchKernelGGL((qgemv_kernel<BITS, LPR, UR, WK>), dim3(grid), dim3(kGemvThreads), lds, st, p);
  return hipGetLastError();
}

template <int BITS, int LPR>
static hipError_t launch_lpr(const GemvProblem& p, const GemvGeom& g, hipStream_t st, size_t lds) {
  if (g.row_unroll == 4 && g.wave_ksplit == 1) return launch_one<BITS, LPR, 4, 1>(p, st, lds);
  if (g.row_unroll == 1 && g.wave_ksplit == 1) return launch_one<BITS, LPR, 1, 1>(p, st, lds);
  if (g.row_unroll == 1 && g.wave_ksplit == 4) return launch_one<BITS, LPR, 1, 4>(p, st, lds);
  if (g.row_unroll == 4 && g.wave_ksplit == 4) return launch_one<BITS, LPR, 4, 4>(p, st, lds);
  return hipErrorInvalidValue;
}

template <int BITS>
static hipError_t launch_bits(const GemvProblem& p, const GemvGeom& g, hipStream_t st) {
  const size_t lds = gemv_lds_bytes(p.k / 64, g);
  switch (g.lanes_per_row) {
    case 1: return launch_lpr<BITS, 1>(p, g, st, lds);
    case 2: return launch_lpr<BITS, 2>(p, g, st, lds);
    case 4: return launch_lpr<BITS, 4>(p, g, st, lds);
    case 8: return launch_lpr<BITS, 8>(p, g, st, lds);
    case 16: return launch_lpr<BITS, 16>(p, g, st, lds);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_qgemv(const GemvProblem& p, int bits, const GemvGeom& g, hipStream_t st) {
  switch (bits) {
    case 2: return launch_bits<2>(p, g, st);
    case 4: return launch_bits<4>(p, g, st);
    case 8: return launch_bits<8>(p, g, st);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS, int LPR>
static hipError_t launch_batched_one(const GemvBlock* blocks, int num_blocks, size_t lds,
                                     hipStream_t st) {
  hipLaunchKernelGGL((qgemv_batched_kernel<BITS, LPR>), dim3(num_blocks), dim3(kGemvThreads), lds,
                     st, blocks);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_batched_bits(const GemvBlock* blocks, int num_blocks, int lpr,
                                      size_t lds, hipStream_t st) {
  switch (lpr) {
    case 1: return launch_batched_one<BITS, 1>(blocks, num_blocks, lds, st);
    case 2: return launch_batched_one<BITS, 2>(blocks, num_blocks, lds, st);
    case 4: return launch_batched_one<BITS, 4>(blocks, num_blocks, lds, st);
    case 8: return launch_batched_one<BITS, 8>(blocks, num_blocks, lds, st);
    case 16: return launch_batched_one<BITS, 16>(blocks, num_blocks, lds, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_qgemv_batched(const GemvBlock* blocks, int num_blocks, int bits,
                                int lanes_per_row, int max_groups, hipStream_t st) {
  GemvGeom g{lanes_per_row, 4, 1, gemv_rows_per_block(lanes_per_row, 4, 1)};
  const size_t lds = gemv_lds_bytes(max_groups, g);
  switch (bits) {
    case 2: return launch_batched_bits<2>(blocks, num_blocks, lanes_per_row, lds, st);
    case 4: return launch_batched_bits<4>(blocks, num_blocks, lanes_per_row, lds, st);
    case 8: return launch_batched_bits<8>(blocks, num_blocks, lanes_per_row, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmm
