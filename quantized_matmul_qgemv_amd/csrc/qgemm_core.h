// Tile core of the prefill GEMM and of the grouped (mixture-of-experts)
// GEMM: y[m, n] = sum_k A[m, k] * W_hat[n, k] with W_hat dequantized to
// fp16 in registers and multiplied on the matrix cores
// (v_mfma_f32_32x32x16_f16, fp32 accumulation).
//
// BaseRT (native-Metal LLM inference on Apple Silicon) §3.4: prefill is a
// tiled GEMM whose arithmetic intensity grows with the sequence length;
// §3.3: dequantization happens inside the inner loop.
//
// Workgroup = 4 wave64s, tile BM x BN (BN = 4 waves x NB x 32).
//   * The 4 waves split the tile's columns: wave w owns columns
//     [w*NB*32, (w+1)*NB*32).  So each weight column is dequantized by
//     exactly one wave (no redundant unpack work).
//   * The weight operand never touches LDS: a lane of a 32x32x16 MFMA
//     supplies 8 consecutive-in-k values of one column, which is one packed
//     word (4-bit), two words (8-bit) or half a word (2-bit).  A lane loads
//     its column's half-group (16 B for 4-bit) with one 128-bit load and
//     dequantizes each word with v_pk_fma_f16(q, s, b): one rounding of the
//     exact s*q + b.
//   * The register unpack yields codes in pair order (see qmm_device.h),
//     not in k order.  A dot product does not care about the order of k
//     inside one MFMA as long as both operands agree, so the A tile is
//     written to LDS with the same order applied inside every 16-wide span
//     of k; the MFMA's A operand is then one ds_read_b128 per lane.
//   * A is double-buffered in LDS (one barrier per pipeline step of GPS
//     groups); the next step's A and packed-B loads are issued before the
//     current step's MFMAs.
//   * The caller chooses the k range, so a tile can be split over k across
//     workgroups (partial tiles are summed by a separate, ordered pass).
#pragma once

#include "qmm_device.h"

namespace qmm {

constexpr int kGemmThreads = 256;

// LDS position p (0..15) inside a 16-wide span of k holds source k = perm16(p).
template <int BITS>
__host__ __device__ constexpr int perm16(int p) {
  // 4-bit: pairs (i, i+4) of each 8-code word; 8-bit: pairs (i, i+2) of each
  // 4-code word; 2-bit: pairs (i, i+8) of one 16-code word.
  return BITS == 4 ? ((p & 8) | ((p & 1) << 2) | ((p & 6) >> 1))
       : BITS == 8 ? ((p & 12) | ((p & 1) << 1) | ((p & 2) >> 1))
                   : (((p & 1) << 3) | (p >> 1));
}

// Permute 16 halves (8 dwords, natural k order) into LDS span order.
template <int BITS>
__device__ __forceinline__ void permute_span(const uint32_t (&in)[8], uint32_t (&out)[8]) {
#pragma unroll
  for (int o = 0; o < 8; ++o) {
    const int k0 = perm16<BITS>(2 * o);
    const int k1 = perm16<BITS>(2 * o + 1);
    const uint32_t lo = (in[k0 >> 1] >> (16 * (k0 & 1))) & 0xFFFFu;
    const uint32_t hi = (in[k1 >> 1] >> (16 * (k1 & 1))) & 0xFFFFu;
    out[o] = lo | (hi << 16);
  }
}

// Packed codes of one column for one lane half (h = lane / 32) and one group.
template <int BITS>
struct BRaw {
  static constexpr int WORDS = Fmt<BITS>::WORDS_PER_GROUP / 2;  // 2, 4 or 8 words
  uint32_t w[WORDS];
  uint16_t s, b;
};

template <int BITS>
__device__ __forceinline__ void load_braw(BRaw<BITS>& r, gptr<uint32_t> wcol, gptr<uint16_t> scol,
                                          gptr<uint16_t> bcol, int g, int h) {
  constexpr int WPG = Fmt<BITS>::WORDS_PER_GROUP;
  gptr<uint32_t> p = wcol + (size_t)g * WPG + h * (WPG / 2);
  if constexpr (BITS == 2) {
    const u32x2 v = *reinterpret_cast<gptr<u32x2>>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < WPG / 2 / 4; ++i) {
      const u32x4 v = reinterpret_cast<gptr<u32x4>>(p)[i];
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
  }
  r.s = scol[g];
  r.b = bcol[g];
}

// B operand (8 fp16 values) of k16 step j (0..3) from a lane's raw half-group.
// The operand is assembled from whole 32-bit pairs (never from extracted
// fp16 vector elements: hipcc for gfx950 has been seen to store the low
// lane where the high lane of a v_pk_fma_f16 result was asked for).
template <int BITS>
__device__ __forceinline__ half8_t b_operand(const BRaw<BITS>& r, int j) {
  const half_t sh = __builtin_bit_cast(half_t, r.s);
  const half_t bh = __builtin_bit_cast(half_t, r.b);
  const half2_t s2{sh, sh}, b2{bh, bh};
  u32x4 o;
  if constexpr (BITS == 4) {
    half2_t d[4];
    dequant_word_f16<4>(r.w[j], s2, b2, d);
    o = u32x4{as_u32(d[0]), as_u32(d[1]), as_u32(d[2]), as_u32(d[3])};
  } else if constexpr (BITS == 8) {
    half2_t d0[2], d1[2];
    dequant_word_f16<8>(r.w[2 * j], s2, b2, d0);
    dequant_word_f16<8>(r.w[2 * j + 1], s2, b2, d1);
    o = u32x4{as_u32(d0[0]), as_u32(d0[1]), as_u32(d1[0]), as_u32(d1[1])};
  } else {
    half2_t d[8];
    dequant_word_f16<2>(r.w[j >> 1], s2, b2, d);
    const int q = (j & 1) * 4;
    o = u32x4{as_u32(d[q]), as_u32(d[q + 1]), as_u32(d[q + 2]), as_u32(d[q + 3])};
  }
  return __builtin_bit_cast(half8_t, o);
}

// Row source for the A tile: dense rows (GEMM) or gathered rows (MoE).
struct ARows {
  const uint16_t* base;  // A matrix, row-major [rows, k]
  int k;
};

// One BM x BN output tile over the k groups [g_begin, g_end).  a_row(i)
// gives the source row of tile row i (already clamped to a valid row);
// c_row(i) gives the output row or -1 to skip; columns are bounded by n.
// Each pipeline step covers GPS groups (GPS*64 values of k): while the
// matrix cores work on step i, the loads of step i+1 are in flight, so a
// larger GPS hides more memory latency per barrier.  (g_end - g_begin) must
// be a multiple of GPS.  lds holds 2 * BM * (64*GPS + 8) halves.
template <int BITS, int BM, int NB, int GPS, typename ARowFn, typename CRowFn>
__device__ __forceinline__ void gemm_tile(const ARows A, ARowFn a_row, CRowFn c_row,
                                          const uint32_t* __restrict__ w_,
                                          const uint16_t* __restrict__ s_,
                                          const uint16_t* __restrict__ b_, float* __restrict__ y_,
                                          int ldy, int n0, int n, int g_begin, int g_end,
                                          uint16_t* lds) {
  constexpr int MB = BM / 32;
  constexpr int SPAN_ROW = 4 * GPS;                  // 16-wide spans per tile row per step
  constexpr int SPANS = BM * SPAN_ROW;
  constexpr int SPT = (SPANS + kGemmThreads - 1) / kGemmThreads;
  constexpr int WPG = Fmt<BITS>::WORDS_PER_GROUP;
  constexpr int AST = 64 * GPS + 8;                  // LDS row stride in halves (16 B pad)
  const gptr<uint32_t> w = to_global(w_);
  const gptr<uint16_t> s = to_global(s_);
  const gptr<uint16_t> b = to_global(b_);
  const gptr_mut<float> y = to_global_mut(y_);
  const gptr<uint16_t> abase = to_global(A.base);
  const int groups = A.k >> 6;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // weight columns of this lane
  gptr<uint32_t> wcol[NB];
  gptr<uint16_t> scol[NB];
  gptr<uint16_t> bcol[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int col = n0 + (wave * NB + nb) * 32 + l32;
    col = col < n ? col : n - 1;
    wcol[nb] = w + (size_t)col * groups * WPG;
    scol[nb] = s + (size_t)col * groups;
    bcol[nb] = b + (size_t)col * groups;
  }

  // A spans of this thread
  gptr<uint16_t> asrc[SPT];
  int aoff[SPT];
  bool aon[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int sp = tid + i * kGemmThreads;
    aon[i] = sp < SPANS;
    const int r = (sp / SPAN_ROW) < BM ? (sp / SPAN_ROW) : BM - 1;
    const int c = sp % SPAN_ROW;
    asrc[i] = abase + (size_t)a_row(r) * A.k + c * 16;
    aoff[i] = r * AST + c * 16;
  }

  float16_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  uint32_t araw[SPT][8];
  BRaw<BITS> braw[GPS][NB];
  auto load_a = [&](int g) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      if (aon[i]) {
        gptr<u32x4> p = reinterpret_cast<gptr<u32x4>>(asrc[i] + (size_t)g * 64);
        const u32x4 v0 = p[0], v1 = p[1];
        araw[i][0] = v0.x; araw[i][1] = v0.y; araw[i][2] = v0.z; araw[i][3] = v0.w;
        araw[i][4] = v1.x; araw[i][5] = v1.y; araw[i][6] = v1.z; araw[i][7] = v1.w;
      }
    }
  };
  auto store_a = [&](int buf) {
    uint16_t* dst = lds + buf * (BM * AST);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      if (aon[i]) {
        uint32_t o[8];
        permute_span<BITS>(araw[i], o);
        u32x4* d = reinterpret_cast<u32x4*>(dst + aoff[i]);
        d[0] = u32x4{o[0], o[1], o[2], o[3]};
        d[1] = u32x4{o[4], o[5], o[6], o[7]};
      }
    }
  };
  auto load_b = [&](int g) {
#pragma unroll
    for (int q = 0; q < GPS; ++q)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        load_braw<BITS>(braw[q][nb], wcol[nb], scol[nb], bcol[nb], g + q, h);
  };

  if (g_begin < g_end) {
    load_a(g_begin);
    load_b(g_begin);
    store_a(0);
  }
  __syncthreads();

  for (int g = g_begin, step = 0; g < g_end; g += GPS, ++step) {
    const int buf = step & 1;
    BRaw<BITS> cur[GPS][NB];
#pragma unroll
    for (int q = 0; q < GPS; ++q)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) cur[q][nb] = braw[q][nb];
    const bool more = g + GPS < g_end;
    if (more) {
      load_a(g + GPS);
      load_b(g + GPS);
    }
    const uint16_t* abuf = lds + buf * (BM * AST);
#pragma unroll
    for (int q = 0; q < GPS; ++q) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8_t bop[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bop[nb] = b_operand<BITS>(cur[q][nb], j);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const half8_t aop = *reinterpret_cast<const half8_t*>(
              abuf + (mb * 32 + l32) * AST + q * 64 + h * 32 + j * 8);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop[nb], acc[mb][nb], 0, 0, 0);
        }
      }
    }
    if (more) store_a(buf ^ 1);
    __syncthreads();
  }

  // epilogue: D[i][j] of a 32x32 block sits in lane (j + 32*((i/4)%2)),
  // register (i/8)*4 + i%4.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = n0 + (wave * NB + nb) * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = mb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        const int row = c_row(i);
        if (row >= 0 && col < n) y[(size_t)row * ldy + col] = acc[mb][nb][r];
      }
    }
  }
}

}  // namespace qmm
