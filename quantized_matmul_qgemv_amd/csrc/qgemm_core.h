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
//   * KW = 2 runs two such groups of 4 waves on the two halves of the
//     tile's k range and adds the halves in LDS at the end: twice the
//     waves per tile (more latency hiding when a grid has few tiles)
//     without the partial tiles and the reduce launch of a k split across
//     workgroups.
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
//     3/5/6-bit weights are unpacked per 8-code chunk in natural order
//     (lane half h at k16 step j takes chunk 4h + j, which is exactly the
//     span of k it reads from LDS), so for them the A tile is stored as is.
//   * Software-pipelined: packed B is loaded 3 steps ahead (registers), A 2
//     steps ahead (registers, then a double-buffered LDS tile); one barrier
//     per step.
//   * The caller chooses the k range, so a tile can be split over k across
//     workgroups (partial tiles are summed in split order afterwards).
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

// Permute 16 halves (8 dwords, natural k order) into LDS span order, one
// v_perm_b32 per output dword.
template <int BITS>
__device__ __forceinline__ void permute_span(const uint32_t (&in)[8], uint32_t (&out)[8]) {
#pragma unroll
  for (int o = 0; o < 8; ++o) {
    const int k0 = perm16<BITS>(2 * o);
    const int k1 = perm16<BITS>(2 * o + 1);
    // selector bytes 0..3 pick from the second source, 4..7 from the first
    const uint32_t lo = (k0 & 1) ? 0x0302u : 0x0100u;
    const uint32_t hi = (k1 & 1) ? 0x07060000u : 0x05040000u;
    out[o] = __builtin_amdgcn_perm(in[k1 >> 1], in[k0 >> 1], lo | hi);
  }
}

// Packed codes of one column for one lane half (h = lane / 32) and one group.
template <int BITS>
struct BRaw {
  static constexpr int WORDS = Fmt<BITS>::WORDS_PER_GROUP / 2;  // 2, 4 or 8 words
  uint32_t w[WORDS];
  uint16_t s, b;
};

// Scale/bias index of lane half h at 64-code step g for groups of gs codes.
__device__ __forceinline__ int sb_index(int g, int h, int gs) {
  return gs == 64 ? g : gs == 32 ? 2 * g + h : (g >> 1);
}

// Weight layouts.  Row-major (wtiled = 0): column c's groups follow each
// other, group g of column c at word (c * G + g) * WPG.  Tile-interleaved
// (wtiled = 1, qmm_repack_tiled): for each block of 32 columns and each
// group, the 32 columns' groups are contiguous, group g of column c at
// word ((c / 32) * G * 32 + g * 32 + c % 32) * WPG, so the 32 columns of a
// wave's weight load are one contiguous run of 32 * WPG words.
__device__ __forceinline__ size_t weight_column_offset(int col, int groups, int wpg, int wtiled) {
  return wtiled ? ((size_t)(col >> 5) * groups * 32 + (col & 31)) * wpg : (size_t)col * groups * wpg;
}

// Scale/bias layouts.  Row-major (stiled = 0): column c's scale and bias of
// scale group i at s[c * SG + i] and b[c * SG + i] (SG = k / gs).
// Interleaved (stiled = 1, qmm_repack_scales_tiled; groups of 64 codes and
// k a multiple of 256): for every block of 32 columns and every quad of 4
// groups, the 32 columns' {s[4q .. 4q+3], b[4q .. 4q+3]} (16 bytes each)
// are contiguous, so a wave's quad loads read 4 whole lines instead of
// parts of 32.  Column c's base (in halves, b == s then):
// ((c / 32) * (G / 4) * 32 + c % 32) * 8; group g's scale at base +
// (g / 4) * 256 + g % 4 and its bias 4 halves later.  The two layouts use
// the same loads (no branch around a load: it would drain the pipeline).
__device__ __forceinline__ size_t scale_column_offset(int col, int sgroups, int stiled) {
  return stiled ? ((size_t)(col >> 5) * (sgroups >> 2) * 32 + (col & 31)) * 8 : (size_t)col * sgroups;
}

__device__ __forceinline__ int scale_quad_offset(int g4, int stiled) { return stiled ? (g4 >> 2) * 256 : g4; }

template <int BITS, bool WITH_SB = true>
__device__ __forceinline__ void load_braw(BRaw<BITS>& r, gptr<uint32_t> wcol, gptr<uint16_t> scol,
                                          gptr<uint16_t> bcol, int g, int h, int gs, int gstride,
                                          int stiled = 0) {
  constexpr int WPG = Fmt<BITS>::WORDS_PER_GROUP;
  gptr<uint32_t> p = wcol + (size_t)g * gstride + h * (WPG / 2);
  if constexpr (BITS == 6) {
    // half a 48-byte group: 8-byte aligned
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const u32x2 v = reinterpret_cast<gptr<u32x2>>(p)[i];
      r.w[2 * i] = v.x; r.w[2 * i + 1] = v.y;
    }
  } else if constexpr (BITS == 3 || BITS == 5) {
    // half a 24- or 40-byte group: 4-byte aligned
#pragma unroll
    for (int i = 0; i < BITS; ++i) r.w[i] = p[i];
  } else if constexpr (BITS == 2) {
    const u32x2 v = *reinterpret_cast<gptr<u32x2>>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < WPG / 2 / 4; ++i) {
      const u32x4 v = reinterpret_cast<gptr<u32x4>>(p)[i];
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
  }
  if constexpr (WITH_SB) {
    const int si = stiled ? (g >> 2) * 256 + (g & 3) : sb_index(g, h, gs);
    r.s = scol[si];
    r.b = bcol[stiled ? si + 4 : si];
  }
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
  } else if constexpr (BITS == 16) {
    // plain fp16 weights: words 4j .. 4j+3 of the lane's 32 k
    o = u32x4{r.w[4 * j], r.w[4 * j + 1], r.w[4 * j + 2], r.w[4 * j + 3]};
  } else if constexpr (BITS == 2) {
    half2_t d[8];
    dequant_word_f16<2>(r.w[j >> 1], s2, b2, d);
    const int q = (j & 1) * 4;
    o = u32x4{as_u32(d[q]), as_u32(d[q + 1]), as_u32(d[q + 2]), as_u32(d[q + 3])};
  } else {
    // chunk j of the lane's half group (BITS words): byte offset BITS*j.
    // j is a constant once the caller's loop is unrolled, so the switch folds.
    constexpr int NW = BRaw<BITS>::WORDS;
    uint32_t vlo, vhi, h[4];
    switch (j) {
      case 0: chunk_window<0, NW>(r.w, vlo, vhi); break;
      case 1: chunk_window<BITS, NW>(r.w, vlo, vhi); break;
      case 2: chunk_window<2 * BITS, NW>(r.w, vlo, vhi); break;
      default: chunk_window<3 * BITS, NW>(r.w, vlo, vhi); break;
    }
    unpack_chunk<BITS>(vlo, vhi, h);
    uint32_t d[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const half2_t q = as_half2(h[t]) - as_half2(chunk_pair<BITS>(t).magic);
      d[t] = as_u32(__builtin_elementwise_fma(q, s2, b2));
    }
    o = u32x4{d[0], d[1], d[2], d[3]};
  }
  return __builtin_bit_cast(half8_t, o);
}

// Row source for the A tile: dense rows (GEMM) or gathered rows (MoE).
struct ARows {
  const uint16_t* base;  // A matrix, row-major [rows, k]
  int k;
};

// One BM x BN output tile over the k groups [g_begin, g_end).  gs is the
// scale group size (32, 64 or 128 codes; SBQ only with 64).  a_row(i)
// gives the source row of tile row i (already clamped to a valid row);
// c_row(i) gives the output row or -1 to skip.  Weight columns start at n0
// and are bounded by n; output column n0 + c goes to y_tile[row * ldy + c]
// (y_tile points at the tile's first column).
//
// Software pipeline, one 64-code group per step (i = step index):
//   * packed B (weights) is loaded 3 steps ahead into a ring of 4 register
//     buffers: it comes straight from HBM and has the longest latency;
//   * A (activations) is loaded 2 steps ahead into 2 register buffers and
//     written to one of 2 LDS slots at the end of the step before its use;
//   * one barrier per step.
// The loop is unrolled by 4 so that every ring index is a compile-time
// constant (register arrays indexed at run time would spill).
// lds holds gemm_lds_halves(BM, NB, KW) halves; the workgroup has
// KW * kGemmThreads threads.
constexpr int kAStride = 72;  // LDS row stride in halves: 64 + 8 pad (144 B)

// LDS of one gemm_tile, in halves: two A slots per k half and, for KW = 2,
// room for the second half's accumulators (4 waves x MB x NB x 16 x 64 floats).
__host__ __device__ constexpr int gemm_lds_halves(int bm, int nb, int kw) {
  return kw * 2 * bm * kAStride > (kw > 1 ? 4 * (bm / 32) * nb * 16 * 64 * 2 : 0)
             ? kw * 2 * bm * kAStride
             : 4 * (bm / 32) * nb * 16 * 64 * 2;
}

//
// SWIGLU (NB = 2): the two column blocks of a wave are the SAME 32 columns of
// two weight sets, gate (w_, s_, b_) and up (w2_, s2_, b2_); the epilogue
// writes h = silu(gate) * up, rounded to fp16, to h_tile[row * ldy + c] for
// the tile's 128 columns (y_tile is unused).
template <int BITS, int BM, int NB, bool SBQ, bool SWIGLU = false, int KW = 1, typename ARowFn,
          typename CRowFn>
__device__ __forceinline__ void gemm_tile(const ARows A, ARowFn a_row, CRowFn c_row,
                                          const uint32_t* __restrict__ w_,
                                          const uint16_t* __restrict__ s_,
                                          const uint16_t* __restrict__ b_, float* __restrict__ y_tile,
                                          int ldy, int n0, int n, int g_begin, int g_end,
                                          uint16_t* lds, int gs = 64,
                                          const uint32_t* __restrict__ w2_ = nullptr,
                                          const uint16_t* __restrict__ s2_ = nullptr,
                                          const uint16_t* __restrict__ b2_ = nullptr,
                                          uint16_t* __restrict__ h_tile = nullptr,
                                          int wtiled = 0, int stiled = 0) {
  static_assert(!SWIGLU || NB == 2, "SwiGLU pairs a gate and an up column block");
  static_assert(KW == 1 || KW == 2, "one or two k halves per workgroup");
  constexpr int MB = BM / 32;
  constexpr int SPANS = BM * 4;  // 16-wide spans of A per step
  constexpr int SPT = (SPANS + kGemmThreads - 1) / kGemmThreads;
  constexpr int WPG = Fmt<BITS>::WORDS_PER_GROUP;
  const int gstride = wtiled ? 32 * WPG : WPG;  // words from one group of a column to the next
  const gptr<uint32_t> w = to_global(w_);
  const gptr<uint16_t> s = to_global(s_);
  const gptr<uint16_t> b = to_global(b_);
  const gptr_mut<float> y = to_global_mut(y_tile);
  const gptr<uint16_t> abase = to_global(A.base);
  const int groups = A.k >> 6;
  const int sgroups = A.k / gs;
  const int tid = KW > 1 ? (int)(threadIdx.x & (kGemmThreads - 1)) : (int)threadIdx.x;  // within its k half
  const int kw = KW > 1 ? (int)(threadIdx.x / kGemmThreads) : 0;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  gptr<uint32_t> wcol[NB];
  gptr<uint16_t> scol[NB];
  gptr<uint16_t> bcol[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int col = SWIGLU ? n0 + wave * 32 + l32 : n0 + (wave * NB + nb) * 32 + l32;
    col = col < n ? col : n - 1;
    const bool second = SWIGLU && nb == 1;
    wcol[nb] = (second ? to_global(w2_) : w) + weight_column_offset(col, groups, WPG, wtiled);
    scol[nb] = (second ? to_global(s2_) : s) + scale_column_offset(col, sgroups, stiled);
    bcol[nb] = stiled ? scol[nb] : (second ? to_global(b2_) : b) + (size_t)col * sgroups;
  }

  // KW = 2: waves 4..7 take the second half of the k range (a multiple of
  // 4 groups when SBQ); both halves run the same number of loop steps (the
  // first half is never the shorter one) and the second half adds its
  // accumulators to the first through LDS at the end.
  int gb = g_begin, ge = g_end, nsteps_all = g_end - g_begin;
  if constexpr (KW > 1) {
    const int G = g_end - g_begin;
    const int h0 = SBQ ? ((G / 4 + 1) / 2) * 4 : (G + 1) / 2;
    gb = kw == 0 ? g_begin : g_begin + h0;
    ge = kw == 0 ? g_begin + h0 : g_end;
    nsteps_all = h0;
  }
  const int nmine = ge - gb;  // steps with work for this half

  gptr<uint16_t> asrc[SPT];
  int aoff[SPT];
  bool aon[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int sp0 = tid + i * kGemmThreads;
    aon[i] = sp0 < SPANS;
    const int sp = sp0 % SPANS;
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

  uint32_t ra[2][SPT][8];   // A register stages
  BRaw<BITS> rb[4][NB];     // B register ring

  // Loads are never predicated: a load under a branch makes the compiler's
  // wait-count bookkeeping fall back to waiting for every outstanding load,
  // which would drain the prefetch pipeline each step.  Threads without a
  // span of their own (BM = 32) reload a valid span and skip the LDS store;
  // steps past the end reload the last group.
  auto load_a = [&](uint32_t (&dst)[SPT][8], int g) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      gptr<u32x4> p = reinterpret_cast<gptr<u32x4>>(asrc[i] + (size_t)g * 64);
      const u32x4 v0 = p[0], v1 = p[1];
      dst[i][0] = v0.x; dst[i][1] = v0.y; dst[i][2] = v0.z; dst[i][3] = v0.w;
      dst[i][4] = v1.x; dst[i][5] = v1.y; dst[i][6] = v1.z; dst[i][7] = v1.w;
    }
  };
  auto store_a = [&](const uint32_t (&src)[SPT][8], int slot) {
    uint16_t* dst = lds + (kw * 2 + slot) * (BM * kAStride);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      if (aon[i]) {
        uint32_t o[8];
        if constexpr (Fmt<BITS>::NATURAL) {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = src[i][e];
        } else {
          permute_span<BITS>(src[i], o);
        }
        u32x4* d = reinterpret_cast<u32x4*>(dst + aoff[i]);
        d[0] = u32x4{o[0], o[1], o[2], o[3]};
        d[1] = u32x4{o[4], o[5], o[6], o[7]};
      }
    }
  };
  auto load_b = [&](BRaw<BITS> (&dst)[NB], int g) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      load_braw<BITS, !SBQ && !Fmt<BITS>::F16W>(dst[nb], wcol[nb], scol[nb], bcol[nb], g, h, gs, gstride,
                                                stiled);
  };
  // SBQ: scales and biases of four consecutive groups come in one 8-byte
  // load per column (a 2-byte load touches as many cache lines as a wide
  // one, so per-group loads made the scale stream as costly as the codes).
  // The caller guarantees g_begin and g_end are multiples of 4.
  u32x2 sqc[NB], bqc[NB], sqn[NB], bqn[NB];
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
  // The A operands of k16 step j+1 are read from LDS while the matrix
  // cores work on step j (two operand buffers), so LDS latency stays off
  // the MFMA issue path.
  auto compute = [&](int slot, const BRaw<BITS> (&cur)[NB]) {
    const uint16_t* abuf = lds + (kw * 2 + slot) * (BM * kAStride) + l32 * kAStride + h * 32;
    half8_t aop[2][MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      aop[0][mb] = *reinterpret_cast<const half8_t*>(abuf + mb * 32 * kAStride);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 3) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          aop[(j + 1) & 1][mb] =
              *reinterpret_cast<const half8_t*>(abuf + mb * 32 * kAStride + (j + 1) * 8);
      }
      half8_t bop[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) bop[nb] = b_operand<BITS>(cur[nb], j);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[j & 1][mb], bop[nb], acc[mb][nb], 0, 0, 0);
    }
  };
  {
  // (a half with no groups clamps to a group just before its range, which
  // lies in [g_begin, g_end), and computes nothing)
  const int nsteps = nsteps_all;
  const int glast = ge - 1;
  auto gclamp = [&](int i) { const int g = gb + i; return g < glast ? g : glast; };
  auto g4clamp = [&](int i) { const int g = gb + i; return g < ge ? g : ge - 4; };
  // prologue: B for steps 0..2, A for steps 0..1, A(0) into LDS slot 0
  if (nsteps > 0) {
    if constexpr (SBQ) load_sbq(sqc, bqc, g4clamp(0));
    load_a(ra[0], gclamp(0));
    load_b(rb[0], gclamp(0));
    load_b(rb[1], gclamp(1));
    load_a(ra[1], gclamp(1));
    load_b(rb[2], gclamp(2));
    store_a(ra[0], 0);
  }
  __syncthreads();

  // step i: B(i+3) -> rb[(i+3)%4], A(i+2) -> ra[i%2]; compute slot i%2 with
  // rb[i%4]; A(i+1) (ra[(i+1)%2]) -> LDS slot (i+1)%2; barrier.  Loads and
  // the store past the last step are harmless repeats of the last group.
  // (Pinning the loads to the top of the step with a scheduling barrier
  // measured 10-17 % slower than leaving the order to the compiler.)
#define QMM_GEMM_STEP(I)                                         \
  {                                                              \
    load_b(rb[((I) + 3) & 3], gclamp(i + (I) + 3));              \
    load_a(ra[(I) & 1], gclamp(i + (I) + 2));                    \
    if (SBQ && (I) == 1) load_sbq(sqn, bqn, g4clamp(i + 4));     \
    set_sb(rb[(I) & 3], (I));                                    \
    if (KW == 1 || i + (I) < nmine) compute((I) & 1, rb[(I) & 3]); \
    store_a(ra[((I) + 1) & 1], ((I) + 1) & 1);                   \
    __syncthreads();                                             \
  }
  int i = 0;
  for (; i + 4 <= nsteps; i += 4) {
    QMM_GEMM_STEP(0)
    QMM_GEMM_STEP(1)
    QMM_GEMM_STEP(2)
    QMM_GEMM_STEP(3)
    if constexpr (SBQ) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) { sqc[nb] = sqn[nb]; bqc[nb] = bqn[nb]; }
    }
  }
  const int rem = nsteps - i;
  if (rem > 0) QMM_GEMM_STEP(0)
  if (rem > 1) QMM_GEMM_STEP(1)
  if (rem > 2) QMM_GEMM_STEP(2)
#undef QMM_GEMM_STEP
  }

  if constexpr (KW > 1) {
    // the second half's accumulators, one 64-float row per register, added
    // into the first half's (the A slots are free after the last barrier)
    float* red = reinterpret_cast<float*>(lds);
    if (kw == 1) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[(((wave * MB + mb) * NB + nb) * 16 + r) * 64 + lane] = acc[mb][nb][r];
    }
    __syncthreads();
    if (kw == 1) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][nb][r] += red[(((wave * MB + mb) * NB + nb) * 16 + r) * 64 + lane];
  }

  // epilogue: D[i][j] of a 32x32 block sits in lane (j + 32*((i/4)%2)),
  // register (i/8)*4 + i%4.
  if constexpr (SWIGLU) {
    const gptr_mut<uint16_t> hp = to_global_mut(h_tile);
    const int lc = wave * 32 + l32;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = mb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        const int row = c_row(i);
        if (row >= 0 && n0 + lc < n) {
          const float g = acc[mb][0][r];
          const float u = acc[mb][1][r];
          const float hv = g / (1.0f + expf(-g)) * u;  // silu(gate) * up
          hp[(size_t)row * ldy + lc] = __builtin_bit_cast(uint16_t, (half_t)hv);
        }
      }
    }
    return;
  }
  // epilogue: D[i][j] of a 32x32 block sits in lane (j + 32*((i/4)%2)),
  // register (i/8)*4 + i%4.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int lc = (wave * NB + nb) * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = mb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        const int row = c_row(i);
        if (row >= 0 && n0 + lc < n) y[(size_t)row * ldy + lc] = acc[mb][nb][r];
      }
    }
  }
}

}  // namespace qmm
