// Load-time quantization and the diagnostic unpack / dequant kernels.
//
// Quantization (asymmetric min/max per group of 32, 64 or 128 along k): per group,
// s = fp16((max - min) / L), b = fp16(min), L = 2^bits - 1, in fp32 with IEEE
// division and round-to-nearest-even; q = clamp(rint((w - b) / s), 0, L)
// using the stored fp16 s and b; q = 0 everywhere when s == 0.  BaseRT
// (native-Metal LLM inference on Apple Silicon) §3.2 prepares all weights
// at model load, so this runs once per weight, not per token.
//
// The diagnostic kernels decode codes and dequantized values with the very
// register routines the GEMV (unpack_word, unpack_chunk) and GEMM
// (dequant_word_f16, and the chunk dequantization) use, so their outputs pin
// those routines bit for bit.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// One thread per (row, group of GS codes).
template <int BITS, int GS>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w,
                                                       uint32_t* __restrict__ words,
                                                       uint16_t* __restrict__ s_out,
                                                       uint16_t* __restrict__ b_out,
                                                       int n, int groups) {
#pragma clang fp contract(off)
  constexpr int WPG = GS * BITS / 32;  // whole words: GS * BITS is a multiple of 32
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)n * groups) return;
  const float* src = w + gid * GS;  // row-major [n, k]: group gid starts at GS*gid
  float v[GS];
#pragma unroll
  for (int i = 0; i < GS / 4; ++i) {
    const float4 f = reinterpret_cast<const float4*>(src)[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < GS; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  const float levels = (float)((1 << BITS) - 1);
  const float s32 = __fdiv_rn(mx - mn, levels);
  const half_t s16 = (half_t)s32;
  const half_t b16 = (half_t)mn;
  const float sf = (float)s16;
  const float bf = (float)b16;
  uint32_t out[WPG];
#pragma unroll
  for (int j = 0; j < WPG; ++j) out[j] = 0u;
#pragma unroll
  for (int i = 0; i < GS; ++i) {
    uint32_t q = 0;
    if (sf != 0.0f) {
      float t = __builtin_rintf(__fdiv_rn(v[i] - bf, sf));
      t = fminf(fmaxf(t, 0.0f), levels);
      q = (uint32_t)t;
    }
    const int bit = i * BITS;
    out[bit >> 5] |= q << (bit & 31);
    if ((bit & 31) + BITS > 32) out[(bit >> 5) + 1] |= q >> (32 - (bit & 31));  // straddles a word
  }
  uint32_t* dst = words + gid * WPG;
#pragma unroll
  for (int j = 0; j < WPG; ++j) dst[j] = out[j];
  s_out[gid] = __builtin_bit_cast(uint16_t, s16);
  b_out[gid] = __builtin_bit_cast(uint16_t, b16);
}

// 3/5/6 bits: the 64-bit window of chunk c (8 codes, BITS bytes, starting
// at byte BITS*c of the flat word array of `words` words).
template <int BITS>
__device__ __forceinline__ void chunk_window_rt(const uint32_t* __restrict__ w, long words, long c,
                                                uint32_t& vlo, uint32_t& vhi) {
  const long byte = (long)BITS * c;
  const long j = byte >> 2;
  const uint32_t o = (uint32_t)(byte & 3);
  // words past the end only feed bytes outside the chunk: clamp
  const long j1 = j + 1 < words ? j + 1 : words - 1;
  const long j2 = j + 2 < words ? j + 2 : words - 1;
  const uint32_t w0 = w[j], w1 = w[j1], w2 = w[j2];
  vlo = __builtin_amdgcn_alignbyte(w1, w0, o);
  vhi = __builtin_amdgcn_alignbyte(w2, w1, o);
}

// One thread per 8-code chunk (3/5/6 bits).
template <int BITS>
__global__ __launch_bounds__(256) void unpack_chunks_kernel(const uint32_t* __restrict__ w,
                                                            uint8_t* __restrict__ codes,
                                                            long words, long chunks) {
  const long c = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  uint32_t vlo, vhi, h[4];
  chunk_window_rt<BITS>(w, words, c, vlo, vhi);
  unpack_chunk<BITS>(vlo, vhi, h);
  uint8_t* dst = codes + c * 8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const half2_t v = as_half2(h[t]);
    dst[2 * t] = (uint8_t)((float)v.x - chunk_magic_value<BITS>(2 * t));
    dst[2 * t + 1] = (uint8_t)((float)v.y - chunk_magic_value<BITS>(2 * t + 1));
  }
}

// One thread per 8-code chunk (3/5/6 bits); a chunk lies in one group.
// fp16 output: v_pk_fma_f16(q, s, b) on q = (magic + q) - magic, as in the
// GEMM's weight operand.
template <int BITS, bool F16>
__global__ __launch_bounds__(256) void dequant_chunks_kernel(const uint32_t* __restrict__ w,
                                                             const uint16_t* __restrict__ s,
                                                             const uint16_t* __restrict__ b,
                                                             void* __restrict__ out, long words,
                                                             long chunks, int gs) {
  const long c = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const long g = c * 8 / gs;  // scale group of the chunk (a chunk never straddles one)
  uint32_t vlo, vhi, h[4];
  chunk_window_rt<BITS>(w, words, c, vlo, vhi);
  unpack_chunk<BITS>(vlo, vhi, h);
  if constexpr (F16) {
    const half_t sh = __builtin_bit_cast(half_t, s[g]);
    const half_t bh = __builtin_bit_cast(half_t, b[g]);
    uint32_t* dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + c * 8);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const half2_t q = as_half2(h[t]) - as_half2(chunk_pair<BITS>(t).magic);
      dst[t] = as_u32(__builtin_elementwise_fma(q, half2_t{sh, sh}, half2_t{bh, bh}));
    }
  } else {
    const float sf = f16_bits_to_f32(s[g]);
    const float bf = f16_bits_to_f32(b[g]);
    float* dst = reinterpret_cast<float*>(out) + c * 8;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const half2_t v = as_half2(h[t]);
      dst[2 * t] = fmaf(sf, (float)v.x - chunk_magic_value<BITS>(2 * t), bf);
      dst[2 * t + 1] = fmaf(sf, (float)v.y - chunk_magic_value<BITS>(2 * t + 1), bf);
    }
  }
}

// One thread per packed word.
template <int BITS>
__global__ __launch_bounds__(256) void unpack_codes_kernel(const uint32_t* __restrict__ w,
                                                           uint8_t* __restrict__ codes,
                                                           long words) {
  using F = Fmt<BITS>;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= words) return;
  uint32_t h[F::PAIRS_PER_WORD];
  unpack_word<BITS>(w[i], h);
  uint8_t* dst = codes + i * F::CODES_PER_WORD;
#pragma unroll
  for (int p = 0; p < F::PAIRS_PER_WORD; ++p) {
    const half2_t v = as_half2(h[p]);
    const float m = magic_value<BITS>(p);
    dst[pair_lo<BITS>(p)] = (uint8_t)((float)v.x - m);
    dst[pair_hi<BITS>(p)] = (uint8_t)((float)v.y - m);
  }
}

// One thread per packed word; every word lies in one scale group.
template <int BITS, bool F16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ w,
                                                      const uint16_t* __restrict__ s,
                                                      const uint16_t* __restrict__ b,
                                                      void* __restrict__ out, long words, int gs) {
  using F = Fmt<BITS>;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= words) return;
  const long k0 = i * F::CODES_PER_WORD;  // global code index
  const long g = k0 / gs;                 // global scale-group index (row-major)
  if constexpr (F16) {
    const half_t sh = __builtin_bit_cast(half_t, s[g]);
    const half_t bh = __builtin_bit_cast(half_t, b[g]);
    half2_t r[F::PAIRS_PER_WORD];
    dequant_word_f16<BITS>(w[i], half2_t{sh, sh}, half2_t{bh, bh}, r);
    // Lanes are taken apart as integers: the halves of an fp16 pair are
    // never extracted as vector elements (see the note on b_operand).
    uint16_t* dst = reinterpret_cast<uint16_t*>(out) + k0;
#pragma unroll
    for (int p = 0; p < F::PAIRS_PER_WORD; ++p) {
      const uint32_t v = as_u32(r[p]);
      dst[pair_lo<BITS>(p)] = (uint16_t)(v & 0xFFFFu);
      dst[pair_hi<BITS>(p)] = (uint16_t)(v >> 16);
    }
  } else {
    const float sf = f16_bits_to_f32(s[g]);
    const float bf = f16_bits_to_f32(b[g]);
    uint32_t h[F::PAIRS_PER_WORD];
    unpack_word<BITS>(w[i], h);
    float* dst = reinterpret_cast<float*>(out) + k0;
#pragma unroll
    for (int p = 0; p < F::PAIRS_PER_WORD; ++p) {
      const half2_t v = as_half2(h[p]);
      const float m = magic_value<BITS>(p);
      dst[pair_lo<BITS>(p)] = fmaf(sf, (float)v.x - m, bf);
      dst[pair_hi<BITS>(p)] = fmaf(sf, (float)v.y - m, bf);
    }
  }
}

static unsigned blocks_for(long items) { return (unsigned)((items + 255) / 256); }

// bf16 weights -> fp16 (load time): the bf16 value widened to fp32 (exact),
// then rounded to fp16 (round to nearest even; beyond fp16's range: +-inf).
// Every bf16 inside fp16's normal range converts exactly (8 significant bits
// into 11).  Two values per thread.
__global__ __launch_bounds__(256) void convert_bf16_kernel(const uint32_t* __restrict__ src,
                                                           uint32_t* __restrict__ dst, long pairs) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= pairs) return;
  const uint32_t v = src[i];
  const float lo = __builtin_bit_cast(float, v << 16);
  const float hi = __builtin_bit_cast(float, v & 0xFFFF0000u);
  const uint32_t l16 = __builtin_bit_cast(uint16_t, (half_t)lo);
  const uint32_t h16 = __builtin_bit_cast(uint16_t, (half_t)hi);
  dst[i] = l16 | (h16 << 16);
}

hipError_t launch_convert_bf16(const uint16_t* src, uint16_t* dst, long count, hipStream_t st) {
  const long pairs = count / 2;
  hipLaunchKernelGGL(convert_bf16_kernel, dim3(blocks_for(pairs)), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), pairs);
  return hipGetLastError();
}

// Tile-interleaved copy of packed weights (one thread per word): group g
// of column c moves from word (c * G + g) * WPG to
// ((c / 32) * G * 32 + g * 32 + c % 32) * WPG.  The GEMM tile core then
// reads the 32 columns of a wave's weight load as one contiguous run.
__global__ __launch_bounds__(256) void repack_tiled_kernel(const uint32_t* __restrict__ src,
                                                           uint32_t* __restrict__ dst, long words,
                                                           int groups, int wpg) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= words) return;
  const long per_col = (long)groups * wpg;
  const long col = i / per_col;
  const long rem = i - col * per_col;
  const long g = rem / wpg;
  const long e = rem - g * wpg;
  dst[(((col >> 5) * groups + g) * 32 + (col & 31)) * wpg + e] = src[i];
}

hipError_t launch_repack_tiled(const uint32_t* w, uint32_t* out, int n, int k, int bits, hipStream_t st) {
  const int wpg = bits * 2;  // words per 64-code group (fp16 weights: 32)
  const long words = (long)n * (k / 64) * wpg;
  hipLaunchKernelGGL(repack_tiled_kernel, dim3(blocks_for(words)), dim3(256), 0, st, w, out, words,
                     k / 64, wpg);
  return hipGetLastError();
}

// Interleaved scales and biases (one thread per column and group of 64):
// column c's scale and bias of group g move from s[c * G + g], b[c * G + g]
// to halves ((c / 32) * (G / 4) * 32 + c % 32) * 8 + (g / 4) * 256 + g % 4
// and 4 halves after it, i.e. for every 32-column block and quad of groups
// the 32 columns' {s[4q .. 4q+3], b[4q .. 4q+3]} lie next to each other.
__global__ __launch_bounds__(256) void repack_scales_tiled_kernel(const uint16_t* __restrict__ s,
                                                                  const uint16_t* __restrict__ b,
                                                                  uint16_t* __restrict__ dst, long count,
                                                                  int groups) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const long col = i / groups;
  const int g = (int)(i - col * groups);
  const long o = (((col >> 5) * (groups >> 2) + (g >> 2)) * 32 + (col & 31)) * 8 + (g & 3);
  dst[o] = s[i];
  dst[o + 4] = b[i];
}

hipError_t launch_repack_scales_tiled(const uint16_t* s, const uint16_t* b, uint16_t* out, int n, int k,
                                      hipStream_t st) {
  const long count = (long)n * (k / 64);
  hipLaunchKernelGGL(repack_scales_tiled_kernel, dim3(blocks_for(count)), dim3(256), 0, st, s, b, out, count,
                     k / 64);
  return hipGetLastError();
}

template <int GS>
static hipError_t launch_quantize_gs(const float* w, uint32_t* words, uint16_t* s, uint16_t* b,
                                     int n, int k, int bits, hipStream_t st) {
  const int groups = k / GS;
  const unsigned grid = blocks_for((long)n * groups);
#define QMM_Q(B) hipLaunchKernelGGL((quantize_kernel<B, GS>), dim3(grid), dim3(256), 0, st, w, words, s, b, n, groups)
  switch (bits) {
    case 2: QMM_Q(2); break;
    case 3: QMM_Q(3); break;
    case 4: QMM_Q(4); break;
    case 5: QMM_Q(5); break;
    case 6: QMM_Q(6); break;
    case 8: QMM_Q(8); break;
    default: return hipErrorInvalidValue;
  }
#undef QMM_Q
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, uint32_t* words, uint16_t* s, uint16_t* b, int n,
                           int k, int bits, int group_size, hipStream_t st) {
  switch (group_size) {
    case 32: return launch_quantize_gs<32>(w, words, s, b, n, k, bits, st);
    case 64: return launch_quantize_gs<64>(w, words, s, b, n, k, bits, st);
    case 128: return launch_quantize_gs<128>(w, words, s, b, n, k, bits, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_unpack_codes(const uint32_t* w, uint8_t* codes, int n, int k, int bits,
                               hipStream_t st) {
  const long words = (long)n * k * bits / 32;
  const unsigned grid = blocks_for(words);
  const long chunks = (long)n * k / 8;
  const unsigned cgrid = blocks_for(chunks);
#define QMM_UC(B) hipLaunchKernelGGL(unpack_chunks_kernel<B>, dim3(cgrid), dim3(256), 0, st, w, codes, words, chunks)
  switch (bits) {
    case 3: QMM_UC(3); break;
    case 5: QMM_UC(5); break;
    case 6: QMM_UC(6); break;
    case 2: hipLaunchKernelGGL(unpack_codes_kernel<2>, dim3(grid), dim3(256), 0, st, w, codes, words); break;
    case 4: hipLaunchKernelGGL(unpack_codes_kernel<4>, dim3(grid), dim3(256), 0, st, w, codes, words); break;
    case 8: hipLaunchKernelGGL(unpack_codes_kernel<8>, dim3(grid), dim3(256), 0, st, w, codes, words); break;
    default: return hipErrorInvalidValue;
  }
#undef QMM_UC
  return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* w, const uint16_t* s, const uint16_t* b, void* out,
                          int out_is_f16, int n, int k, int bits, int gs, hipStream_t st) {
  const long words = (long)n * k * bits / 32;
  const unsigned grid = blocks_for(words);
  const long chunks = (long)n * k / 8;
  const unsigned cgrid = blocks_for(chunks);
#define QMM_DQ(B, H) hipLaunchKernelGGL((dequant_kernel<B, H>), dim3(grid), dim3(256), 0, st, w, s, b, out, words, gs)
#define QMM_DQC(B, H) hipLaunchKernelGGL((dequant_chunks_kernel<B, H>), dim3(cgrid), dim3(256), 0, st, w, s, b, out, words, chunks, gs)
  if (out_is_f16) {
    switch (bits) {
      case 2: QMM_DQ(2, true); break;
      case 3: QMM_DQC(3, true); break;
      case 4: QMM_DQ(4, true); break;
      case 5: QMM_DQC(5, true); break;
      case 6: QMM_DQC(6, true); break;
      case 8: QMM_DQ(8, true); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (bits) {
      case 2: QMM_DQ(2, false); break;
      case 3: QMM_DQC(3, false); break;
      case 4: QMM_DQ(4, false); break;
      case 5: QMM_DQC(5, false); break;
      case 6: QMM_DQC(6, false); break;
      case 8: QMM_DQ(8, false); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef QMM_DQ
#undef QMM_DQC
  return hipGetLastError();
}

}  // namespace qmm
