// Load-time quantization and the diagnostic unpack / dequant kernels.
//
// Quantization (asymmetric min/max per group of 64 along k): per group,
// s = fp16((max - min) / L), b = fp16(min), L = 2^bits - 1, in fp32 with IEEE
// division and round-to-nearest-even; q = clamp(rint((w - b) / s), 0, L)
// using the stored fp16 s and b; q = 0 everywhere when s == 0.  BaseRT
// (native-Metal LLM inference on Apple Silicon) §3.2 prepares all weights
// at model load, so this runs once per weight, not per token.
//
// The diagnostic kernels decode codes and dequantized values with the very
// register routines the GEMV (unpack_word) and GEMM (dequant_word_f16) use,
// so their outputs pin those routines bit for bit.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// One thread per (row, group).
template <int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w,
                                                       uint32_t* __restrict__ words,
                                                       uint16_t* __restrict__ s_out,
                                                       uint16_t* __restrict__ b_out,
                                                       int n, int groups) {
#pragma clang fp contract(off)
  using F = Fmt<BITS>;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)n * groups) return;
  const float* src = w + gid * 64;  // row-major [n, k]: group gid starts at 64*gid
  float v[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 f = reinterpret_cast<const float4*>(src)[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 64; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  const float levels = (float)((1 << BITS) - 1);
  const float s32 = __fdiv_rn(mx - mn, levels);
  const half_t s16 = (half_t)s32;
  const half_t b16 = (half_t)mn;
  const float sf = (float)s16;
  const float bf = (float)b16;
  uint32_t out[F::WORDS_PER_GROUP];
#pragma unroll
  for (int j = 0; j < F::WORDS_PER_GROUP; ++j) out[j] = 0u;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    uint32_t q = 0;
    if (sf != 0.0f) {
      float t = __builtin_rintf(__fdiv_rn(v[i] - bf, sf));
      t = fminf(fmaxf(t, 0.0f), levels);
      q = (uint32_t)t;
    }
    out[(i * BITS) >> 5] |= q << ((i * BITS) & 31);
  }
  uint32_t* dst = words + gid * F::WORDS_PER_GROUP;
#pragma unroll
  for (int j = 0; j < F::WORDS_PER_GROUP; ++j) dst[j] = out[j];
  s_out[gid] = __builtin_bit_cast(uint16_t, s16);
  b_out[gid] = __builtin_bit_cast(uint16_t, b16);
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

// One thread per packed word; every word lies in one group.
template <int BITS, bool F16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ w,
                                                      const uint16_t* __restrict__ s,
                                                      const uint16_t* __restrict__ b,
                                                      void* __restrict__ out, long words) {
  using F = Fmt<BITS>;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= words) return;
  const long g = i / F::WORDS_PER_GROUP;  // global group index (row-major)
  const long k0 = i * F::CODES_PER_WORD;  // global code index
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

hipError_t launch_quantize(const float* w, uint32_t* words, uint16_t* s, uint16_t* b, int n,
                           int k, int bits, hipStream_t st) {
  const int groups = k / 64;
  const unsigned grid = blocks_for((long)n * groups);
  switch (bits) {
    case 2: hipLaunchKernelGGL(quantize_kernel<2>, dim3(grid), dim3(256), 0, st, w, words, s, b, n, groups); break;
    case 4: hipLaunchKernelGGL(quantize_kernel<4>, dim3(grid), dim3(256), 0, st, w, words, s, b, n, groups); break;
    case 8: hipLaunchKernelGGL(quantize_kernel<8>, dim3(grid), dim3(256), 0, st, w, words, s, b, n, groups); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_unpack_codes(const uint32_t* w, uint8_t* codes, int n, int k, int bits,
                               hipStream_t st) {
  const long words = (long)n * k * bits / 32;
  const unsigned grid = blocks_for(words);
  switch (bits) {
    case 2: hipLaunchKernelGGL(unpack_codes_kernel<2>, dim3(grid), dim3(256), 0, st, w, codes, words); break;
    case 4: hipLaunchKernelGGL(unpack_codes_kernel<4>, dim3(grid), dim3(256), 0, st, w, codes, words); break;
    case 8: hipLaunchKernelGGL(unpack_codes_kernel<8>, dim3(grid), dim3(256), 0, st, w, codes, words); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* w, const uint16_t* s, const uint16_t* b, void* out,
                          int out_is_f16, int n, int k, int bits, hipStream_t st) {
  const long words = (long)n * k * bits / 32;
  const unsigned grid = blocks_for(words);
#define QMM_DQ(B, H) hipLaunchKernelGGL((dequant_kernel<B, H>), dim3(grid), dim3(256), 0, st, w, s, b, out, words)
  if (out_is_f16) {
    switch (bits) {
      case 2: QMM_DQ(2, true); break;
      case 4: QMM_DQ(4, true); break;
      case 8: QMM_DQ(8, true); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (bits) {
      case 2: QMM_DQ(2, false); break;
      case 4: QMM_DQ(4, false); break;
      case 8: QMM_DQ(8, false); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef QMM_DQ
  return hipGetLastError();
}

}  // namespace qmm
