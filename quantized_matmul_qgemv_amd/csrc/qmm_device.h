// Device-side building blocks shared by the GEMV, GEMM and diagnostic
// kernels: the packed-code format, the register unpack and small helpers.
//
// Unpack.  A packed uint32 word holds C = 32 / BITS codes, code i in bits
// [BITS*i, BITS*i + BITS) (low code first along k).  The register unpack
// turns one word into C/2 fp16 pairs without any integer-to-float
// conversion: a code placed in the low mantissa bits of an fp16 whose
// exponent field is fixed reads as (magic + code), exactly.  Pair p holds
// codes (p, p + C/2) of the word, so one AND-OR with a mask that repeats in
// both 16-bit halves extracts two codes at once:
//
//   code bit offset o inside its 16-bit half   magic (fp16 bits)  value
//   o = 0                                      0x6400             1024 + q
//   o = 2                                      0x5C00              256 + q
//   o = 4                                      0x5400               64 + q
//   o = 6                                      0x4C00               16 + q
//
// (an fp16 in [2^e, 2^(e+1)) has ulp 2^(e-10); putting q at bit o needs ulp
// 2^-o, so the magic is 2^(10-o)).  For 8-bit codes a byte permute moves
// bytes 1 and 3 to the low byte of each half.
//
// Consumers must pair activations the same way: pair p of a word spanning
// k0 .. k0+C-1 multiplies (x[k0+p], x[k0+p+C/2]).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int BITS>
struct Fmt {
  static_assert((BITS >= 2 && BITS <= 8 && BITS != 7) || BITS == 16,
                "supported widths: 2, 3, 4, 5, 6, 8 and 16 (unquantized fp16 weights)");
  // 3-, 5- and 6-bit codes straddle word boundaries and are unpacked per
  // 8-code chunk (BITS bytes, see unpack_chunk); the others per word.
  static constexpr bool CHUNKED = (32 % BITS) != 0;
  // 16: the weights are plain fp16 values (two per word, low half first);
  // there are no codes, scales or biases.
  static constexpr bool F16W = BITS == 16;
  // weight pairs in natural k order (no activation permutation needed)
  static constexpr bool NATURAL = CHUNKED || F16W;
  static constexpr int CODES_PER_WORD = CHUNKED ? 0 : 32 / BITS;
  static constexpr int PAIRS_PER_WORD = CODES_PER_WORD / 2;
  static constexpr int WORDS_PER_GROUP = 64 * BITS / 32;  // group of 64 codes
  static constexpr int VEC4_PER_GROUP = WORDS_PER_GROUP / 4 > 0 ? WORDS_PER_GROUP / 4 : 1;
  static constexpr int GROUP_BYTES = WORDS_PER_GROUP * 4;
  static constexpr int PAIRS_PER_GROUP = 32;
};

// Offset added by the magic exponent to the code of pair p.
template <int BITS>
__host__ __device__ constexpr float magic_value(int p) {
  return BITS == 8 ? 1024.0f
       : BITS == 4 ? ((p & 1) ? 64.0f : 1024.0f)
       : (p & 3) == 0 ? 1024.0f : (p & 3) == 1 ? 256.0f : (p & 3) == 2 ? 64.0f : 16.0f;
}

template <int BITS>
__host__ __device__ constexpr uint32_t magic_bits(int p) {
  return BITS == 8 ? 0x64006400u
       : BITS == 4 ? ((p & 1) ? 0x54005400u : 0x64006400u)
       : (p & 3) == 0 ? 0x64006400u : (p & 3) == 1 ? 0x5C005C00u
       : (p & 3) == 2 ? 0x54005400u : 0x4C004C00u;
}

// (a & mask) | magic in ONE instruction.  The compiler splits it into
// v_and_b32 + v_or_b32 with literal operands (a VOP3 instruction on this
// chip takes no literal and at most one SGPR), doubling the unpack cost;
// here the mask sits in an SGPR and the magic in a VGPR, both hoisted out
// of every loop by the compiler.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(magic));
  return d;
}

// One packed word -> PAIRS_PER_WORD fp16 pairs (as raw 32-bit patterns),
// pair p = (magic + code p, magic + code p + C/2).
template <int BITS>
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t (&h)[Fmt<BITS>::PAIRS_PER_WORD]) {
  if constexpr (BITS == 4) {
    const uint32_t w8 = w >> 8;
    h[0] = and_or(w, 0x000F000Fu, 0x64006400u);
    h[1] = and_or(w, 0x00F000F0u, 0x54005400u);
    h[2] = and_or(w8, 0x000F000Fu, 0x64006400u);
    h[3] = and_or(w8, 0x00F000F0u, 0x54005400u);
  } else if constexpr (BITS == 8) {
    // bytes: D.b[i] = {S0:S1}.b[sel.b[i]], S1 = bytes 0..3, S0 = bytes 4..7
    h[0] = and_or(w, 0x00FF00FFu, 0x64006400u);
    h[1] = __builtin_amdgcn_perm(w, 0x64646464u, 0x00070005u);
  } else if constexpr (BITS == 16) {
    h[0] = w;  // already an fp16 pair
  } else {
    const uint32_t w8 = w >> 8;
    h[0] = and_or(w, 0x00030003u, 0x64006400u);
    h[1] = and_or(w, 0x000C000Cu, 0x5C005C00u);
    h[2] = and_or(w, 0x00300030u, 0x54005400u);
    h[3] = and_or(w, 0x00C000C0u, 0x4C004C00u);
    h[4] = and_or(w8, 0x00030003u, 0x64006400u);
    h[5] = and_or(w8, 0x000C000Cu, 0x5C005C00u);
    h[6] = and_or(w8, 0x00300030u, 0x54005400u);
    h[7] = and_or(w8, 0x00C000C0u, 0x4C004C00u);
  }
}

// Position (within the word's span of C codes) of the low / high element of pair p.
template <int BITS>
__host__ __device__ constexpr int pair_lo(int p) { return p; }
template <int BITS>
__host__ __device__ constexpr int pair_hi(int p) { return p + Fmt<BITS>::CODES_PER_WORD / 2; }

// Pointers that reach a kernel inside a structure loaded from memory are
// generic (flat) pointers to the compiler; flat loads count against both
// the vector-memory and the LDS wait counters, so every LDS wait would also
// wait for all outstanding weight loads.  Casting to the global address
// space restores global_load/global_store.
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;
template <typename T>
using gptr_mut = __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ gptr<T> to_global(const T* p) { return (gptr<T>)(p); }
template <typename T>
__device__ __forceinline__ gptr_mut<T> to_global_mut(T* p) { return (gptr_mut<T>)(p); }

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(half_t, b);
}

// acc + a.x*b.x + a.y*b.y with fp32 accumulation (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(as_half2(a), as_half2(b), acc, false);
}

// ---------------------------------------------------------------------------
// 3-, 5- and 6-bit codes: chunk unpack.
//
// Eight consecutive codes fill exactly BITS bytes, so every 8-code chunk
// starts on a byte boundary and its codes sit at the same bit positions in
// every chunk.  Let V be the 64-bit value whose low byte is the chunk's
// first byte (vlo = V[31:0], vhi = V[63:32]) and S = (V >> 4)[31:0].  Pair t
// of a chunk is (code 2t, code 2t+1), in natural k order.  Each code is
// read through a 16-bit window that starts on a byte of V (or of S when the
// code would otherwise sit too high in its window): the code must lie at a
// bit offset o with o + BITS <= 10 so that the magic fp16 2^(10-o), whose
// ulp is 2^-o, reads as (2^(10-o) + code) exactly.  One v_perm_b32 moves
// both windows into place (lo window -> bits 0..15, hi window -> bits
// 16..31), one AND-OR keeps the two code fields and sets the magics.
//
// Code positions (bit offset inside the chunk) and windows:
//   3-bit: 0,3,6,9,12,15,18,21          all from V bytes 0..3
//   5-bit: 0,5,10,15,20,25,30,35         codes 3 and 6 from S (offset 7 and 6 in V are too high)
//   6-bit: 0,6,12,18,24,30,36,42         codes 1 and 5 from S
// Table entries: {src0, src1, selector, mask, magic}; v_perm_b32(src0,
// src1, sel) takes byte i of the result from byte sel.b[i] of the 8-byte
// value src0:src1 (bytes 0..3 = src1, 4..7 = src0).
struct ChunkPair {
  int src0, src1;  // 0 = vlo, 1 = vhi, 2 = S
  uint32_t sel, mask, magic;
};

template <int BITS>
__host__ __device__ constexpr ChunkPair chunk_pair(int t) {
  if constexpr (BITS == 3) {
    return t == 0 ? ChunkPair{0, 0, 0x01000100u, 0x00380007u, 0x58006400u}   // offsets 0 | 3
         : t == 1 ? ChunkPair{0, 0, 0x02010100u, 0x000E01C0u, 0x60004C00u}   // 6 | 1
         : t == 2 ? ChunkPair{0, 0, 0x02010201u, 0x03800070u, 0x48005400u}   // 4 | 7
                  : ChunkPair{0, 0, 0x03020302u, 0x00E0001Cu, 0x50005C00u};  // 2 | 5
  } else if constexpr (BITS == 5) {
    return t == 0 ? ChunkPair{0, 0, 0x01000100u, 0x03E0001Fu, 0x50006400u}   // 0 | 5
         : t == 1 ? ChunkPair{2, 0, 0x05050101u, 0x00F8007Cu, 0x58005C00u}   // 2 | S:3
         : t == 2 ? ChunkPair{0, 0, 0x03030302u, 0x003E01F0u, 0x60005400u}   // 4 | 1
                  : ChunkPair{1, 2, 0x04040303u, 0x00F8007Cu, 0x58005C00u};  // S:2 | 3
  } else {
    static_assert(BITS == 6, "chunk tables exist for 3, 5 and 6 bits");
    return t == 0 ? ChunkPair{2, 0, 0x04040000u, 0x00FC003Fu, 0x5C006400u}   // 0 | S:2
         : t == 1 ? ChunkPair{0, 0, 0x02020201u, 0x00FC03F0u, 0x5C005400u}   // 4 | 2
         : t == 2 ? ChunkPair{2, 0, 0x07070303u, 0x00FC003Fu, 0x5C006400u}   // 0 | S:2
                  : ChunkPair{1, 1, 0x01010100u, 0x00FC03F0u, 0x5C005400u};  // 4 | 2
  }
}

// Offset added by the magic to code c (0..7) of a chunk.
template <int BITS>
__host__ __device__ constexpr float chunk_magic_value(int c) {
  const uint32_t m = (c & 1) ? (chunk_pair<BITS>(c >> 1).magic >> 16) : (chunk_pair<BITS>(c >> 1).magic & 0xFFFFu);
  // fp16 with zero mantissa: 2^(exponent - 15)
  return (float)(1u << ((m >> 10) - 15));
}

// The 64-bit window V of the chunk starting at byte SB of w[0 .. NW).
// Words past the end are never needed for the code bits (they are clamped
// to the last word and only feed masked-off bytes).
template <int SB, int NW>
__device__ __forceinline__ void chunk_window(const uint32_t* w, uint32_t& vlo, uint32_t& vhi) {
  constexpr int j = SB / 4, o = SB % 4;
  constexpr int j1 = j + 1 < NW ? j + 1 : NW - 1;
  constexpr int j2 = j + 2 < NW ? j + 2 : NW - 1;
  if constexpr (o == 0) {
    vlo = w[j];
    vhi = w[j1];
  } else {
    vlo = __builtin_amdgcn_alignbyte(w[j1], w[j], o);
    vhi = __builtin_amdgcn_alignbyte(w[j2], w[j1], o);
  }
}

// One 8-code chunk -> 4 fp16 pairs (raw 32-bit patterns),
// pair t = (magic + code 2t, magic + code 2t+1).
template <int BITS>
__device__ __forceinline__ void unpack_chunk(uint32_t vlo, uint32_t vhi, uint32_t (&h)[4]) {
  const uint32_t sv = __builtin_amdgcn_alignbit(vhi, vlo, 4);
  auto pick = [&](int i) { return i == 0 ? vlo : i == 1 ? vhi : sv; };
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const ChunkPair c = chunk_pair<BITS>(t);
    h[t] = and_or(__builtin_amdgcn_perm(pick(c.src0), pick(c.src1), c.sel), c.mask, c.magic);
  }
}

}  // namespace qmm

namespace qmm {

// Dequantize one packed word to fp16 in register-pair order:
// out[p] = fp16(s * q + b) for the two codes of pair p, computed as
// v_pk_fma_f16(q, s, b) with q = (magic + q) - magic (exact), so each value
// is the exact s*q + b rounded once to fp16.
template <int BITS>
__device__ __forceinline__ void dequant_word_f16(uint32_t w, half2_t s2, half2_t b2,
                                                 half2_t (&out)[Fmt<BITS>::PAIRS_PER_WORD]) {
  uint32_t h[Fmt<BITS>::PAIRS_PER_WORD];
  unpack_word<BITS>(w, h);
#pragma unroll
  for (int p = 0; p < Fmt<BITS>::PAIRS_PER_WORD; ++p) {
    const half2_t q = as_half2(h[p]) - as_half2(magic_bits<BITS>(p));
    out[p] = __builtin_elementwise_fma(q, s2, b2);
  }
}

}  // namespace qmm
