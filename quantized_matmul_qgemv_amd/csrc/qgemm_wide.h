// Wide tile of the prefill GEMM: 256 x 256 outputs per workgroup, one
// workgroup per CU.  Same arithmetic as gemm_tile in qgemm_core.h (weights
// dequantized to fp16 in registers with one rounding of s*q + b, fp32
// accumulation on v_mfma_f32_32x32x16_f16); what changes is the shape of
// the work on the CU:
//
//   * 4 waves, wave w owns columns [w*64, w*64+64) and all 256 rows: each
//     dequantized weight operand feeds 8 MFMAs, so the unpack costs half as
//     much per MFMA as in the 128-row tile, and no column is unpacked twice.
//   * 256 accumulator registers per lane (8 x 2 blocks of 32x32): one wave
//     per SIMD, with the 512-entry register file to itself.
//   * A (activations) goes global -> registers -> LDS through a ring of 3
//     LDS stages: step i multiplies stage i%3, writes step i+2 into stage
//     (i+2)%3 and, before its barrier, already reads the first operands of
//     step i+1, so the barrier never leaves the matrix core without work.
//
// BaseRT (native-Metal LLM inference on Apple Silicon) §3.4 (prefill as a
// tiled GEMM whose efficiency grows with the tile) and §3.3 (dequantization
// inside the inner loop).
#pragma once

#include "qgemm_core.h"

namespace qmm {

constexpr int kWideBM = 256;
constexpr int kWideStages = 3;
constexpr int kWideLdsHalves = kWideStages * kWideBM * kAStride;  // 110,592 bytes

template <int BITS, bool SBQ, typename ARowFn, typename CRowFn>
__device__ __forceinline__ void gemm_tile_wide(const ARows A, ARowFn a_row, CRowFn c_row,
                                               const uint32_t* __restrict__ w_,
                                               const uint16_t* __restrict__ s_,
                                               const uint16_t* __restrict__ b_,
                                               float* __restrict__ y_tile, int ldy, int n0, int n,
                                               int g_begin, int g_end, uint16_t* lds, int gs = 64,
                                               int wtiled = 0, int stiled = 0) {
  constexpr int BM = kWideBM;
  constexpr int MB = BM / 32;
  constexpr int NB = 2;
  constexpr int SPT = BM * 4 / kGemmThreads;  // 16-wide spans of A per thread per step
  constexpr int WPG = Fmt<BITS>::WORDS_PER_GROUP;
  constexpr int SLOT = BM * kAStride;
  const int gstride = wtiled ? 32 * WPG : WPG;
  const gptr<uint32_t> w = to_global(w_);
  const gptr<uint16_t> s = to_global(s_);
  const gptr<uint16_t> b = to_global(b_);
  const gptr_mut<float> y = to_global_mut(y_tile);
  const gptr<uint16_t> abase = to_global(A.base);
  const int groups = A.k >> 6;
  const int sgroups = A.k / gs;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  gptr<uint32_t> wcol[NB];
  gptr<uint16_t> scol[NB];
  gptr<uint16_t> bcol[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int col = n0 + (wave * NB + nb) * 32 + l32;
    col = col < n ? col : n - 1;
    wcol[nb] = w + weight_column_offset(col, groups, WPG, wtiled);
    scol[nb] = s + scale_column_offset(col, sgroups, stiled);
    bcol[nb] = stiled ? scol[nb] : b + (size_t)col * sgroups;
  }
  gptr<uint16_t> asrc[SPT];
  int aoff[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int sp = tid + i * kGemmThreads;
    const int r = sp >> 2;
    const int c = sp & 3;
    asrc[i] = abase + (size_t)a_row(r) * A.k + c * 16;
    aoff[i] = r * kAStride + c * 16;
  }

  float16_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  uint32_t ra[SPT][8];
  BRaw<BITS> rb[4][NB];
  half8_t aop[2][MB];
  u32x2 sqc[NB], bqc[NB], sqn[NB], bqn[NB];

  auto load_a = [&](uint32_t (&dst)[SPT][8], int g) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      gptr<u32x4> p = reinterpret_cast<gptr<u32x4>>(asrc[i] + (size_t)g * 64);
      const u32x4 v0 = p[0], v1 = p[1];
      dst[i][0] = v0.x; dst[i][1] = v0.y; dst[i][2] = v0.z; dst[i][3] = v0.w;
      dst[i][4] = v1.x; dst[i][5] = v1.y; dst[i][6] = v1.z; dst[i][7] = v1.w;
    }
  };
  auto store_a = [&](const uint32_t (&src)[SPT][8], uint16_t* slot) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      uint32_t o[8];
      if constexpr (Fmt<BITS>::NATURAL) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = src[i][e];
      } else {
        permute_span<BITS>(src[i], o);
      }
      u32x4* d = reinterpret_cast<u32x4*>(slot + aoff[i]);
      d[0] = u32x4{o[0], o[1], o[2], o[3]};
      d[1] = u32x4{o[4], o[5], o[6], o[7]};
    }
  };
  auto load_b = [&](BRaw<BITS> (&dst)[NB], int g) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      load_braw<BITS, !SBQ && !Fmt<BITS>::F16W>(dst[nb], wcol[nb], scol[nb], bcol[nb], g, h, gs, gstride,
                                                stiled);
  };
  auto load_sbq = [&](u32x2 (&sq)[NB], u32x2 (&bq)[NB], int g4) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int so = scale_quad_offset(g4, stiled);
      sq[nb] = *reinterpret_cast<gptr<u32x2>>(scol[nb] + so);
      bq[nb] = *reinterpret_cast<gptr<u32x2>>(bcol[nb] + (stiled ? so + 4 : so));
    }
  };
  auto set_sb = [&](BRaw<BITS> (&cur)[NB], int q) {
    if constexpr (SBQ) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t sw = (q >> 1) ? sqc[nb].y : sqc[nb].x;
        const uint32_t bw = (q >> 1) ? bqc[nb].y : bqc[nb].x;
        cur[nb].s = (uint16_t)(sw >> (16 * (q & 1)));
        cur[nb].b = (uint16_t)(bw >> (16 * (q & 1)));
      }
    }
  };
  // Operand reads: a lane reads row l32 of each 32-row block, k offset
  // 32*h + 8*j of the (permuted) 64-wide stage.
  const int aread = l32 * kAStride + h * 32;
  auto read_a = [&](half8_t (&dst)[MB], const uint16_t* slot, int j) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      dst[mb] = *reinterpret_cast<const half8_t*>(slot + aread + mb * 32 * kAStride + j * 8);
  };

  const int nsteps = g_end - g_begin;
  const int glast = g_end - 1;
  auto gclamp = [&](int i) { const int g = g_begin + i; return g < glast ? g : glast; };
  auto g4clamp = [&](int i) { const int g = g_begin + i; return g < g_end ? g : g_end - 4; };

  // prologue: A(0), A(1) into stages 0, 1; A(2) in registers; B(0..2)
  if constexpr (SBQ) load_sbq(sqc, bqc, g_begin);
  load_a(ra, gclamp(0));
  load_b(rb[0], gclamp(0));
  load_b(rb[1], gclamp(1));
  store_a(ra, lds);
  load_a(ra, gclamp(1));
  load_b(rb[2], gclamp(2));
  store_a(ra, lds + SLOT);
  load_a(ra, gclamp(2));
  __syncthreads();
  read_a(aop[0], lds, 0);

  // Step i (I = i % 4): registers ra hold A(i+2), rb[I] holds B(i).
  //   load B(i+3) -> rb[(I+3)&3];
  //   multiply stage i%3 (operands for j = 0 are already in aop[0]);
  //   after the first k16 block: store A(i+2) into stage (i+2)%3, then
  //   load A(i+3) into ra;
  //   read operands j = 0 of stage (i+1)%3; barrier.
  // Loads past the last step repeat the last group (never predicated: a
  // load under a branch makes the wait-count bookkeeping drain all loads).
  uint16_t* cur = lds;
  uint16_t* nxt = lds + SLOT;
  uint16_t* fut = lds + 2 * SLOT;
#define QMM_WIDE_STEP(I)                                                                   \
  {                                                                                        \
    load_b(rb[((I) + 3) & 3], gclamp(i + (I) + 3));                                        \
    if (SBQ && (I) == 1) load_sbq(sqn, bqn, g4clamp(i + 4));                               \
    set_sb(rb[(I)], (I));                                                                  \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                        \
      if (j < 3) read_a(aop[(j + 1) & 1], cur, j + 1);                                     \
      half8_t bop[NB];                                                                     \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) bop[nb] = b_operand<BITS>(rb[(I)][nb], j); \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                    \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                    \
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[j & 1][mb], bop[nb], acc[mb][nb], 0, 0, 0); \
      if (j == 0) { store_a(ra, fut); load_a(ra, gclamp(i + (I) + 3)); }                   \
    }                                                                                      \
    read_a(aop[0], nxt, 0);                                                                \
    __syncthreads();                                                                       \
    uint16_t* t_ = cur; cur = nxt; nxt = fut; fut = t_;                                    \
  }
  int i = 0;
  for (; i + 4 <= nsteps; i += 4) {
    QMM_WIDE_STEP(0)
    QMM_WIDE_STEP(1)
    QMM_WIDE_STEP(2)
    QMM_WIDE_STEP(3)
    if constexpr (SBQ) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) { sqc[nb] = sqn[nb]; bqc[nb] = bqn[nb]; }
    }
  }
  const int rem = nsteps - i;
  if (rem > 0) QMM_WIDE_STEP(0)
  if (rem > 1) QMM_WIDE_STEP(1)
  if (rem > 2) QMM_WIDE_STEP(2)
#undef QMM_WIDE_STEP

  // epilogue: D[i][j] of a 32x32 block sits in lane (j + 32*((i/4)%2)),
  // register (i/8)*4 + i%4.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int lc = (wave * NB + nb) * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row_i = mb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        const int row = c_row(row_i);
        if (row >= 0 && n0 + lc < n) y[(size_t)row * ldy + lc] = acc[mb][nb][r];
      }
    }
  }
}

}  // namespace qmm
