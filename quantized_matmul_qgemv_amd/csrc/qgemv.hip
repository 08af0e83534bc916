// Decode GEMV over group-quantized weights (BaseRT, native-Metal LLM
// inference on Apple Silicon, §3.3: one GEMV kernel per quantization
// format, dequantization folded into the inner loop).
//
// y[n] = sum_g ( s[n,g] * sum_{k in g} q[n,k] x[k]  +  b[n,g] * sum_{k in g} x[k] )
//
// The kernel is HBM-bound: every packed weight byte is read exactly once.
// Work decomposition (one workgroup = 4 wave64s):
//   * a "unit" is one 64-code group of one row: GROUP_BYTES (8 * bits:
//     16/24/32/40/48/64 B for 2/3/4/5/6/8 bits) of codes plus one fp16
//     scale and one fp16 bias;
//   * LPR consecutive lanes share a row; lane lr takes the row's groups
//     lr, lr + LPR, lr + 2*LPR, ...  so one wave-wide 128-bit load covers
//     64/LPR rows with contiguous, fully used 16-byte pieces (4- and 8-bit
//     codes in 64-code scale groups and fp16 weights: a lane takes a half,
//     a quarter or an eighth of two, four or eight groups per step instead,
//     so that each of its loads reads whole contiguous lines; see
//     gemv_block);
//   * each lane keeps UR rows in flight (128 bytes of codes per lane for 4
//     and 8 bits, 64 for 2 bits), and
//     the loads of the next step are issued before the current step is
//     consumed (two register buffers used alternately);
//   * a workgroup can run several passes of rows over the same activations
//     (the prefetch then runs across pass boundaries); one pass per
//     workgroup measured best, since the dispatcher balances short
//     workgroups across CUs better than long ones;
//   * for small n, WK waves of a workgroup split a row's groups and meet in
//     LDS (deterministic, no atomics).
// Activations are staged once per workgroup in LDS in "paired" order (the
// order the register unpack produces codes in, see qmm_device.h), together
// with two per-group constants:
//     C[g] = sum_{k in g} magic(k) * x[k]       X[g] = sum_{k in g} x[k]
// so that   sum_k q_k x_k = dot(magic + q, x) - C[g]   needs no per-code
// subtraction: each packed 4-bit word costs one shift, four AND-ORs and
// four v_dot2_f32_f16.  3-, 5- and 6-bit codes straddle words; they are
// read as window pairs (WinPairs below), one AND-OR per pair from a 32-bit
// window of the group's words, and the staging writes x in that pair order.
#include <type_traits>

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
  static constexpr int ROWS = WR * UR * RPW;   // rows per workgroup pass
};

// a.x*b.x + a.y*b.y with fp32 accumulation, starting from zero: the
// three-operand form with an inline 0, where the compiler's own choice (the
// two-operand form that accumulates in place) first needs a move of 0.
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b) {
  float d;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// Window pairing of 3-, 5- and 6-bit codes in the GEMV.  A 32-code half of
// a 64-code group is BITS words; code c sits at bit BITS*c.  Each pair
// (c1, c2) is read from a 32-bit window of the half starting at bit s: c1 at
// offset o1 = BITS*c1 - s of the low 16 bits, c2 at o2 = BITS*c2 - s - 16 of
// the high 16 bits, both with o + BITS <= 10, so that ONE AND-OR with the
// magic 2^(10-o) per half turns the window into the fp16 pair
// (2^(10-o1) + q1, 2^(10-o2) + q2).  Windows at multiples of 32 bits are
// the words themselves; the others cost one funnel shift (or one shift
// inside the last word).  The 16 (s, c1, c2) of each width were chosen by an
// exact-cover search over all windows for the fewest shifts, then the fewest
// distinct (o1, o2) (the magics held in registers):
//   3 bits: 4 shifts per half, 72 VALU per 64 codes (102 for the byte-permute
//           chunk unpack of qmm_device.h), 7 magics;
//   5 bits: 12 shifts, 88 VALU (about 115), 4 magics;
//   6 bits: 10 shifts, 84 VALU (about 111), 3 magics.
// Slot p of a half holds the pair below; the staging writes (x[c1], x[c2])
// there.
struct WinPair {
  int s, c1, c2;
};

template <int BITS>
struct WinPairs;
template <>
struct WinPairs<3> {
  static constexpr WinPair p[16] = {{0, 0, 6},   {0, 1, 7},   {6, 2, 8},   {6, 3, 9},
                                    {12, 4, 10}, {12, 5, 11}, {32, 12, 17}, {32, 13, 18},
                                    {41, 14, 19}, {41, 15, 20}, {41, 16, 21}, {64, 22, 28},
                                    {64, 23, 27}, {71, 24, 29}, {71, 25, 30}, {71, 26, 31}};
};
template <>
struct WinPairs<5> {
  static constexpr WinPair p[16] = {{0, 0, 4},    {5, 1, 5},    {10, 2, 6},   {15, 3, 7},
                                    {36, 8, 11},  {43, 9, 12},  {49, 10, 14}, {64, 13, 17},
                                    {73, 15, 18}, {78, 16, 19}, {96, 20, 23}, {103, 21, 24},
                                    {108, 22, 25}, {128, 26, 29}, {131, 27, 30}, {138, 28, 31}};
};
template <>
struct WinPairs<6> {
  static constexpr WinPair p[16] = {{0, 0, 3},    {6, 1, 4},    {12, 2, 5},   {32, 6, 8},
                                    {42, 7, 10},  {52, 9, 12},  {64, 11, 14}, {74, 13, 15},
                                    {96, 16, 19}, {102, 17, 20}, {108, 18, 21}, {128, 22, 24},
                                    {136, 23, 26}, {150, 25, 28}, {160, 27, 30}, {170, 29, 31}};
};

template <int BITS>
constexpr bool win_pairs() { return BITS == 3 || BITS == 5 || BITS == 6; }
static_assert(win_pairs<3>() == Fmt<3>::CHUNKED && win_pairs<5>() == Fmt<5>::CHUNKED &&
                  win_pairs<6>() == Fmt<6>::CHUNKED && !Fmt<2>::CHUNKED && !Fmt<4>::CHUNKED && !Fmt<8>::CHUNKED,
              "every width whose codes straddle words is read as window pairs");
template <int BITS>
constexpr int win_o1(const WinPair& p) { return BITS * p.c1 - p.s; }
template <int BITS>
constexpr int win_o2(const WinPair& p) { return BITS * p.c2 - p.s - 16; }

template <int BITS>
constexpr bool win_table_ok() {
  bool seen[32] = {};
  for (const WinPair& p : WinPairs<BITS>::p) {
    const int o1 = win_o1<BITS>(p), o2 = win_o2<BITS>(p);
    if (o1 < 0 || o1 + BITS > 10 || o2 < 0 || o2 + BITS > 10) return false;
    if (p.c1 < 0 || p.c1 > 31 || p.c2 < 0 || p.c2 > 31 || seen[p.c1] || seen[p.c2]) return false;
    seen[p.c1] = seen[p.c2] = true;
  }
  return true;
}
static_assert(win_table_ok<3>() && win_table_ok<5>() && win_table_ok<6>(),
              "window pairs must cover the half once, each code inside its window");

// Code bits kept and magic exponents set by the AND-OR of a pair.
template <int BITS>
constexpr uint32_t win_mask(const WinPair& p) {
  constexpr uint32_t m = (1u << BITS) - 1;
  return (m << win_o1<BITS>(p)) | (m << (16 + win_o2<BITS>(p)));
}
template <int BITS>
constexpr uint32_t win_magic(const WinPair& p) {
  return ((uint32_t)(25 - win_o1<BITS>(p)) << 10) | ((uint32_t)(25 - win_o2<BITS>(p)) << 26);
}

// Window of the half w[0 .. NW) starting at bit S (bits past the half read
// 0 and are masked off).
template <int S, int NW>
__device__ __forceinline__ uint32_t half_window(const uint32_t* w) {
  constexpr int j = S / 32, r = S % 32;
  if constexpr (r == 0) return w[j];
  else if constexpr (j + 1 < NW) return __builtin_amdgcn_alignbit(w[j + 1], w[j], r);
  else return w[j] >> r;
}

// Pair slot P of a half: window, AND-OR into the fp16 pair, dot product
// with the staged activations (the first slot of a half starts from zero).
template <int BITS, int P>
__device__ __forceinline__ void win_slot(const uint32_t* w, uint32_t x, float& a) {
  constexpr WinPair p = WinPairs<BITS>::p[P];
  const uint32_t hp = and_or(half_window<p.s, BITS>(w), win_mask<BITS>(p), win_magic<BITS>(p));
  a = P == 0 ? dot2_first(hp, x) : dot2(hp, x, a);
}

// Stage x[0 .. 64*groups) into LDS: paired halves plus (C[g], X[g]).  Four
// consecutive threads share a group (16 codes each), so the staging that
// every workgroup waits for at its barrier is short.  It is split in two:
// stage_x_load issues the activation loads (before the weight loads, so
// that waiting for x never waits for the weight stream, loads completing
// in order) and stage_x_store pairs, sums and writes them to LDS.  For
// 3-bit weights a thread builds 8 pair slots of one 32-code half, whose
// codes lie anywhere in the half, so it holds the whole half (32 codes).
constexpr int kXRounds = 1;  // quarter-groups per thread held in registers (k <= 4096)

template <int BITS>
constexpr int x_words() { return win_pairs<BITS>() ? 16 : 8; }  // activation dwords per thread

template <int BITS>
struct XStage {
  uint32_t d[kXRounds][x_words<BITS>()];
};

// The activations a staging thread t needs: its quarter (16 codes), or for
// 3-bit weights the 32-code half its quarter belongs to.
template <int BITS>
__device__ __forceinline__ void load_quarter(gptr<uint16_t> x, int t, uint32_t (&d)[x_words<BITS>()]) {
  constexpr int NV = x_words<BITS>() / 4;
  const size_t off = win_pairs<BITS>() ? (size_t)(t >> 2) * 64 + ((t >> 1) & 1) * 32 : (size_t)(t >> 2) * 64 + (t & 3) * 16;
  gptr<u32x4> src = reinterpret_cast<gptr<u32x4>>(x + off);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const u32x4 q = src[v];
    d[4 * v] = q.x; d[4 * v + 1] = q.y; d[4 * v + 2] = q.z; d[4 * v + 3] = q.w;
  }
}

template <int BITS>
__device__ __forceinline__ void stage_x_load(gptr<uint16_t> x, int groups, XStage<BITS>& xs) {
#pragma unroll
  for (int r = 0; r < kXRounds; ++r) {
    int t = threadIdx.x + r * kGemvThreads;
    const int last = 4 * groups - 1;
    t = t < last ? t : last;  // unpredicated: repeat the last quarter
    load_quarter<BITS>(x, t, xs.d[r]);
  }
}

// fp16 bits of activation c from dwords holding activations in natural order.
template <int N>
__device__ __forceinline__ uint32_t x_half(const uint32_t (&d)[N], int c) {
  return (d[c >> 1] >> (16 * (c & 1))) & 0xFFFFu;
}

// Pair slots and (C, X) shares of one staging thread: out[0..7] are the 8
// dwords it writes at pair index part*8 of its group.
template <int BITS>
__device__ __forceinline__ void build_quarter(const uint32_t (&d)[x_words<BITS>()], int part, uint32_t (&out)[8],
                                              float& csum, float& xsum) {
  using F = Fmt<BITS>;
  csum = 0.0f;
  xsum = 0.0f;
  if constexpr (F::F16W) {
    // fp16 weights: x in natural order, no magic offsets (C = 0)
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = d[i];
  } else if constexpr (win_pairs<BITS>()) {
    // slots sub*8 .. sub*8+7 of the thread's half (sub = part & 1)
    const bool sub = (part & 1) != 0;
    auto slot = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr WinPair p0 = WinPairs<BITS>::p[j], p1 = WinPairs<BITS>::p[8 + j];
      constexpr float ml0 = (float)(1 << (10 - win_o1<BITS>(p0))), ml1 = (float)(1 << (10 - win_o1<BITS>(p1)));
      constexpr float mh0 = (float)(1 << (10 - win_o2<BITS>(p0))), mh1 = (float)(1 << (10 - win_o2<BITS>(p1)));
      const uint32_t v0 = x_half(d, p0.c1) | (x_half(d, p0.c2) << 16);
      const uint32_t v1 = x_half(d, p1.c1) | (x_half(d, p1.c2) << 16);
      out[j] = sub ? v1 : v0;
      const float xl = f16_bits_to_f32((uint16_t)(out[j] & 0xFFFFu));
      const float xh = f16_bits_to_f32((uint16_t)(out[j] >> 16));
      csum += (sub ? ml1 : ml0) * xl;
      csum += (sub ? mh1 : mh0) * xh;
      xsum += xl;
      xsum += xh;
    };
    slot(std::integral_constant<int, 0>{});
    slot(std::integral_constant<int, 1>{});
    slot(std::integral_constant<int, 2>{});
    slot(std::integral_constant<int, 3>{});
    slot(std::integral_constant<int, 4>{});
    slot(std::integral_constant<int, 5>{});
    slot(std::integral_constant<int, 6>{});
    slot(std::integral_constant<int, 7>{});
  } else {
    constexpr int C = F::CODES_PER_WORD;
    constexpr int PPW = F::PAIRS_PER_WORD;
    constexpr int WPQ = 16 / C > 0 ? 16 / C : 1;  // words per quarter group
    static_assert(16 % C == 0, "a quarter group must hold whole words");
#pragma unroll
    for (int wd = 0; wd < WPQ; ++wd) {
#pragma unroll
      for (int p = 0; p < PPW; ++p) {
        const int klo = wd * C + pair_lo<BITS>(p);
        const int khi = wd * C + pair_hi<BITS>(p);
        const uint32_t lo = x_half(d, klo);
        const uint32_t hi = x_half(d, khi);
        out[wd * PPW + p] = lo | (hi << 16);
        const float xl = f16_bits_to_f32((uint16_t)lo);
        const float xh = f16_bits_to_f32((uint16_t)hi);
        csum += magic_value<BITS>(p) * xl;
        csum += magic_value<BITS>(p) * xh;
        xsum += xl;
        xsum += xh;
      }
    }
  }
}

// One quarter group -> its pair slots in LDS and its share of (C, X).
template <int BITS, int GS>
__device__ __forceinline__ void stage_quarter(const uint32_t (&d)[x_words<BITS>()], int g, int part, bool on,
                                              unsigned char* xp, float* cx) {
  float csum, xsum;
  uint32_t out[8];
  build_quarter<BITS>(d, part, out, csum, xsum);
  if (on) {
    // pairs of this quarter: 8 dwords at pair index part*8 of the group
    u32x4* dst = reinterpret_cast<u32x4*>(xp + (size_t)g * kXStride + part * 32);
    dst[0] = u32x4{out[0], out[1], out[2], out[3]};
    dst[1] = u32x4{out[4], out[5], out[6], out[7]};
  }
  csum += __shfl_xor(csum, 1);
  xsum += __shfl_xor(xsum, 1);
  if constexpr (GS == 32) {
    // (C, X) of each 32-code half: {C_lo, X_lo, C_hi, X_hi} per group
    if (on && (part & 1) == 0) reinterpret_cast<float2*>(cx)[2 * g + (part >> 1)] = make_float2(csum, xsum);
  } else {
    csum += __shfl_xor(csum, 2);
    xsum += __shfl_xor(xsum, 2);
    if (on && part == 0) reinterpret_cast<float2*>(cx)[g] = make_float2(csum, xsum);
  }
}

template <int BITS, int GS>
__device__ __forceinline__ void stage_x_store(gptr<uint16_t> x, int groups, const XStage<BITS>& xs,
                                              unsigned char* xp, float* cx, bool stager) {
  const int quarters = 4 * groups;
#pragma unroll
  for (int r = 0; r < kXRounds; ++r) {
    const int t = threadIdx.x + r * kGemvThreads;
    if (r > 0 || stager) stage_quarter<BITS, GS>(xs.d[r], t >> 2, t & 3, t < quarters, xp, cx);
  }
  // quarters beyond the register rounds (k > 4096): load and stage directly
  const int rounds = (quarters + kGemvThreads - 1) / kGemvThreads;  // uniform
  for (int r = kXRounds; r < rounds; ++r) {
    const int t0 = threadIdx.x + r * kGemvThreads;
    const int t = t0 < quarters ? t0 : quarters - 1;
    uint32_t d[x_words<BITS>()];
    load_quarter<BITS>(x, t, d);
    stage_quarter<BITS, GS>(d, t0 >> 2, t0 & 3, t0 < quarters, xp, cx);
  }
}

// Moves between lanes of one 16-lane row through the DPP operand modifier
// (no LDS round trip): lane i reads lane i ^ 8 (row_ror:8), i ^ 7
// (row_half_mirror), i ^ 2 and i ^ 1 (quad permutes).
constexpr int kDppRor8 = 0x128, kDppHalfMirror = 0x141, kDppXor2 = 0x4E, kDppXor1 = 0xB1;

template <int CTRL>
__device__ __forceinline__ float dpp_read(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sums each of UR per-row partials over the 16 lanes of a row (lane lr =
// 0..15 of the row's lanes) with the exchanges transposed: the first two
// exchanges each halve the values a lane carries (a lane keeps the rows its
// partner does not), so every lane ends with the total of row
// lr / (16 / UR), held by 16 / UR lanes.  For UR = 4 that is 11 VALU
// instructions instead of 16 additions and 16 LDS permutes.
template <int UR>
__device__ __forceinline__ float row_sum16(const float (&a)[UR], int lr) {
  static_assert(UR == 1 || UR == 2 || UR == 4, "row_sum16 takes 1, 2 or 4 rows");
  const bool b3 = (lr & 8) != 0, b2 = (lr & 4) != 0;
  float v;
  if constexpr (UR == 4) {
    // i ^ 8: lanes with bit 3 clear keep rows 0, 1, the others rows 2, 3
    const float k0 = (b3 ? a[2] : a[0]) + dpp_read<kDppRor8>(b3 ? a[0] : a[2]);
    const float k1 = (b3 ? a[3] : a[1]) + dpp_read<kDppRor8>(b3 ? a[1] : a[3]);
    // i ^ 7 flips bit 2: bit 2 picks one row of the pair
    v = (b2 ? k1 : k0) + dpp_read<kDppHalfMirror>(b2 ? k0 : k1);
  } else if constexpr (UR == 2) {
    const float k = (b3 ? a[1] : a[0]) + dpp_read<kDppRor8>(b3 ? a[0] : a[1]);
    v = k + dpp_read<kDppHalfMirror>(k);
  } else {
    v = a[0] + dpp_read<kDppRor8>(a[0]);
    v += dpp_read<kDppHalfMirror>(v);
  }
  // lanes {i, i^8, i^7, i^15} are summed; i ^ 2 and i ^ 1 add the other 12
  v += dpp_read<kDppXor2>(v);
  v += dpp_read<kDppXor1>(v);
  return v;
}

// Partial dot products a[v] of part q (= lane % NP) of NP groups, held by
// the NP consecutive lanes of a cluster: returns the cluster's total for
// group v = q, with the exchanges transposed (a lane keeps the groups its
// partner does not): one quad permute for NP = 2, two for NP = 4.
template <int NP>
__device__ __forceinline__ float cluster_sum(const float (&a)[NP], int q) {
  static_assert(NP == 2 || NP == 4, "clusters of 2 or 4 lanes");
  if constexpr (NP == 2) {
    return (q ? a[1] : a[0]) + dpp_read<kDppXor1>(q ? a[0] : a[1]);
  } else {
    // i ^ 2: lanes with bit 1 clear keep groups 0, 1, the others 2, 3
    const bool b1 = (q & 2) != 0;
    const float k0 = (b1 ? a[2] : a[0]) + dpp_read<kDppXor2>(b1 ? a[0] : a[2]);
    const float k1 = (b1 ? a[3] : a[1]) + dpp_read<kDppXor2>(b1 ? a[1] : a[3]);
    return ((q & 1) ? k1 : k0) + dpp_read<kDppXor1>((q & 1) ? k0 : k1);
  }
}

// Weight-stream loads (codes, scales and biases), non-temporal (NT) where
// every wave-wide load consumes whole 128-byte lines: the 2-bit groups (one
// 16-byte load per lane) and the split-group lanes below (4 and 8 bits, fp16).  The
// stream is read once and need not stay in L2; a plain read kernel over the
// same bytes streams 7-10 % faster with such loads.  Where a lane reads its
// group with several loads, each covering part of every line (3, 5 and 6
// bits, and 4 and 8 bits with whole groups per lane), the same policy
// measured 5-38 % slower, so those keep ordinary loads.
template <bool NT, typename T>
__device__ __forceinline__ T stream_load(gptr<T> p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Register buffer of one step: UR rows x one group per lane.  3/5/6-bit
// groups (24/40/48 bytes) are loaded with 8-byte loads unless 16-byte
// aligned (6 bits).
template <int BITS>
struct GroupLoad {
  static constexpr int BYTES = Fmt<BITS>::GROUP_BYTES;
  static constexpr int VB = BYTES % 16 == 0 ? 16 : 8;  // bytes per load
  static constexpr int NV = BYTES / VB;                // loads per group
};

// SBN scale/bias pairs per 64-code group: 2 for groups of 32, else 1.
template <int BITS, int UR, int SBN, bool CH = Fmt<BITS>::CHUNKED>
struct StepBuf {
  u32x4 w[UR][Fmt<BITS>::VEC4_PER_GROUP];
  uint16_t s[UR][SBN], b[UR][SBN];
};

template <int BITS, int UR, int SBN>
struct StepBuf<BITS, UR, SBN, true> {
  uint32_t w[UR][Fmt<BITS>::WORDS_PER_GROUP];
  uint16_t s[UR][SBN], b[UR][SBN];
};

// GS: codes per scale/bias group (32, 64 or 128); the kernel works in
// 64-code units throughout, with two scale groups per unit for GS = 32 and
// one scale group per two units for GS = 128.
template <int BITS, int LPR, int UR, int WK, int GS>
__device__ __forceinline__ void gemv_block(const GemvProblem& P, int row0, int nrows,
                                           unsigned char* smem) {
  using F = Fmt<BITS>;
  using Cfg = GemvCfg<BITS, LPR, UR, WK>;
  constexpr int V4 = F::VEC4_PER_GROUP;
  constexpr int WPG = F::WORDS_PER_GROUP;
  constexpr int PPW = F::PAIRS_PER_WORD;
  // Split-group lanes (4- and 8-bit codes in 64-code scale groups, and
  // fp16 weights): a group is NP = 2, 4 or 8 sixteen-byte pieces.  At a k-step over groups
  // sb .. sb+LPR-1 of a row, lane lr loads pieces NP*sb + LPR*v + lr
  // (v < NP): part q = lr % NP of groups sb + (LPR/NP)*v + lr/NP, so each
  // wave-wide load reads whole contiguous lines (with one group per lane,
  // each of a lane's NP loads took every NP-th piece of the lines).  The NP
  // lanes of a cluster (lr / NP) then hold every part of NP groups; DPP
  // exchanges (cluster_sum) leave each lane the whole dot product of group
  // v = q, and each lane folds that one group (fp16 weights have no fold:
  // every piece goes straight into the row sum).
  constexpr int NP = F::GROUP_BYTES / 16;
  constexpr bool SPLIT = ((BITS == 4 || BITS == 8) && GS == 64 || F::F16W) && LPR % NP == 0;
  constexpr bool NT = BITS == 2 || SPLIT;
  constexpr int SBN = GS == 32 ? 2 : 1;
  using Buf = StepBuf<BITS, UR, SBN>;

  const int groups = P.k >> 6;
  const int sgroups = P.k / GS;  // scale groups per row
  unsigned char* xp = smem;
  float* cx = reinterpret_cast<float*>(smem + (size_t)groups * kXStride);  // 2 or 4 floats per unit
  float* red = cx + (size_t)groups * 2 * SBN;

  const gptr<uint32_t> W = to_global(P.w);
  const gptr<uint16_t> S = to_global(P.s);
  const gptr<uint16_t> B = to_global(P.b);
  const gptr_mut<float> Y = to_global_mut(P.y);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave / WK;
  const int wk = wave % WK;
  const int slot = lane / LPR;
  const int lr = lane % LPR;
  const int T = groups / LPR;
  const int tcount = T > wk ? (T - wk + WK - 1) / WK : 0;  // k-steps of this wave per pass
  const int npass = (nrows + Cfg::ROWS - 1) / Cfg::ROWS;
  const int nsteps = npass * tcount;
  const int row_end = (row0 + nrows < P.n ? row0 + nrows : P.n);
  const int lane_row = row0 + wr * UR * Cfg::RPW + slot;  // + pass*ROWS + u*RPW
  const size_t rstride = (size_t)groups * WPG;

  // step -> (pass, t): incremental counters for the issuing side
  int ip = 0, it = 0;
  auto issue = [&](Buf& bf) {
    int g = (wk + it * WK) * LPR + lr;
    g = g < groups ? g : groups - 1;  // only a wave with no k-steps (WK > 1) goes past
    if constexpr (SPLIT) {
      int sb = (wk + it * WK) * LPR;
      sb = sb < groups ? sb : groups - LPR;  // (LPR divides groups)
      const int jm = sb + (LPR / NP) * (lr % NP) + lr / NP;  // the group this lane folds
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        int r = lane_row + ip * Cfg::ROWS + u * Cfg::RPW;
        r = r < row_end ? r : row_end - 1;
        const gptr<u32x4> src = reinterpret_cast<gptr<u32x4>>(W + (size_t)r * rstride) + (size_t)NP * sb + lr;
#pragma unroll
        for (int v = 0; v < NP; ++v) bf.w[u][v] = stream_load<NT>(src + LPR * v);
        if constexpr (!F::F16W) {
          bf.s[u][0] = stream_load<NT>(S + (size_t)r * sgroups + jm);
          bf.b[u][0] = stream_load<NT>(B + (size_t)r * sgroups + jm);
        }
      }
      if (++it == tcount) { it = 0; ++ip; }
      return;
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      int r = lane_row + ip * Cfg::ROWS + u * Cfg::RPW;
      r = r < row_end ? r : row_end - 1;
      if constexpr (F::CHUNKED) {
        using GL = GroupLoad<BITS>;
        if constexpr (GL::VB == 16) {
          gptr<u32x4> src = reinterpret_cast<gptr<u32x4>>(W + (size_t)r * rstride + (size_t)g * WPG);
#pragma unroll
          for (int v = 0; v < GL::NV; ++v) {
            const u32x4 t = stream_load<NT>(src + v);
            bf.w[u][4 * v] = t.x; bf.w[u][4 * v + 1] = t.y; bf.w[u][4 * v + 2] = t.z; bf.w[u][4 * v + 3] = t.w;
          }
        } else {
          gptr<u32x2> src = reinterpret_cast<gptr<u32x2>>(W + (size_t)r * rstride + (size_t)g * WPG);
#pragma unroll
          for (int v = 0; v < GL::NV; ++v) {
            const u32x2 t = stream_load<NT>(src + v);
            bf.w[u][2 * v] = t.x; bf.w[u][2 * v + 1] = t.y;
          }
        }
      } else {
        gptr<u32x4> src = reinterpret_cast<gptr<u32x4>>(W + (size_t)r * rstride + (size_t)g * WPG);
#pragma unroll
        for (int v = 0; v < V4; ++v) bf.w[u][v] = stream_load<NT>(src + v);
      }
      if constexpr (!F::F16W) {
#pragma unroll
        for (int q = 0; q < SBN; ++q) {
          const size_t si = (size_t)r * sgroups + (GS == 32 ? 2 * g + q : GS == 128 ? (g >> 1) : g);
          bf.s[u][q] = stream_load<NT>(S + si);
          bf.b[u][q] = stream_load<NT>(B + si);
        }
      }
    }
    if (++it == tcount) { it = 0; ++ip; }
  };

  float acc[UR];
#pragma unroll
  for (int u = 0; u < UR; ++u) acc[u] = 0.0f;

  int cp = 0, ct = 0;  // consuming side
  auto consume = [&](const Buf& bf) {
    const int g = (wk + ct * WK) * LPR + lr;
    const unsigned char* xg = xp + (size_t)g * kXStride;
    float a0[UR], a1[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) a0[u] = a1[u] = 0.0f;
    if constexpr (SPLIT && F::F16W) {
      // fp16 weights have no per-group fold: every piece's dot product goes
      // straight into the row sum (x in natural order, 16 bytes per piece)
      const int sb = (wk + ct * WK) * LPR;
      const int q = lr % NP, c = lr / NP;
#pragma unroll
      for (int v = 0; v < NP; ++v) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xp + (size_t)(sb + (LPR / NP) * v + c) * kXStride + 16 * q);
#pragma unroll
        for (int u = 0; u < UR; ++u) {
          const u32x4 wv = bf.w[u][v];
          a0[u] = v == 0 ? dot2_first(wv.x, xv.x) : dot2(wv.x, xv.x, a0[u]);
          a1[u] = v == 0 ? dot2_first(wv.y, xv.y) : dot2(wv.y, xv.y, a1[u]);
          a0[u] = dot2(wv.z, xv.z, a0[u]);
          a1[u] = dot2(wv.w, xv.w, a1[u]);
        }
      }
    } else if constexpr (SPLIT) {
      // part q of groups sb + (LPR/NP)*v + c, v < NP (their x pairs: bytes
      // (128/NP)*q .. of each group's staging), one partial sum per group
      const int sb = (wk + ct * WK) * LPR;
      const int q = lr % NP, c = lr / NP;
      float a[UR][NP];
#pragma unroll
      for (int v = 0; v < NP; ++v) {
        const unsigned char* xv = xp + (size_t)(sb + (LPR / NP) * v + c) * kXStride + (128 / NP) * q;
#pragma unroll
        for (int jw = 0; jw < 4; ++jw) {
          uint32_t xr[PPW];
          if constexpr (PPW == 2) {
            const uint2 t = *reinterpret_cast<const uint2*>(xv + 8 * jw);
            xr[0] = t.x; xr[1] = t.y;
          } else {
            const u32x4 t = *reinterpret_cast<const u32x4*>(xv + 16 * jw);
            xr[0] = t.x; xr[1] = t.y; xr[2] = t.z; xr[3] = t.w;
          }
#pragma unroll
          for (int u = 0; u < UR; ++u) {
            const u32x4 wv = bf.w[u][v];
            const uint32_t word = jw == 0 ? wv.x : jw == 1 ? wv.y : jw == 2 ? wv.z : wv.w;
            uint32_t h[PPW];
            unpack_word<BITS>(word, h);
#pragma unroll
            for (int p = 0; p < PPW; ++p)
              a[u][v] = jw == 0 && p == 0 ? dot2_first(h[p], xr[p]) : dot2(h[p], xr[p], a[u][v]);
          }
        }
      }
      const float2 cxy = reinterpret_cast<const float2*>(cx)[sb + (LPR / NP) * q + c];
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const float dot = cluster_sum<NP>(a[u], q);
        const float s = f16_bits_to_f32(bf.s[u][0]);
        const float b = f16_bits_to_f32(bf.b[u][0]);
        acc[u] = fmaf(s, dot - cxy.x, fmaf(b, cxy.y, acc[u]));
      }
    } else if constexpr (F::F16W) {
      // 16 bytes of weights (8 fp16) against 16 bytes of x at a time
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const u32x4 xv = reinterpret_cast<const u32x4*>(xg)[q];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
          const u32x4 wv = bf.w[u][q];
          a0[u] = q == 0 ? dot2_first(wv.x, xv.x) : dot2(wv.x, xv.x, a0[u]);
          a1[u] = q == 0 ? dot2_first(wv.y, xv.y) : dot2(wv.y, xv.y, a1[u]);
          a0[u] = dot2(wv.z, xv.z, a0[u]);
          a1[u] = dot2(wv.w, xv.w, a1[u]);
        }
      }
    } else if constexpr (win_pairs<BITS>()) {
      // window pairs (WinPairs): half h of the group is words BITS*h ..
      // BITS*h+BITS-1 and its 16 pair slots are dwords 16h .. 16h+15 of the
      // group's x; the two halves accumulate apart (they are the two scale
      // groups of 32)
      auto half = [&](auto hc) {
        constexpr int h = decltype(hc)::value;
        auto quad = [&](auto qc) {
          constexpr int q = decltype(qc)::value;
          const u32x4 xv = reinterpret_cast<const u32x4*>(xg)[4 * h + q];
          const uint32_t xr[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int u = 0; u < UR; ++u) {
            float& a = h == 0 ? a0[u] : a1[u];
            const uint32_t* w = bf.w[u] + BITS * h;
            win_slot<BITS, 4 * q + 0>(w, xr[0], a);
            win_slot<BITS, 4 * q + 1>(w, xr[1], a);
            win_slot<BITS, 4 * q + 2>(w, xr[2], a);
            win_slot<BITS, 4 * q + 3>(w, xr[3], a);
          }
        };
        quad(std::integral_constant<int, 0>{});
        quad(std::integral_constant<int, 1>{});
        quad(std::integral_constant<int, 2>{});
        quad(std::integral_constant<int, 3>{});
      };
      half(std::integral_constant<int, 0>{});
      half(std::integral_constant<int, 1>{});
    } else {
    // word-major: the activation pairs of one word are read from LDS once
    // and used for all UR rows, so only PPW of them are live at a time
#pragma unroll
    for (int j = 0; j < WPG; ++j) {
      uint32_t xr[PPW];
      if constexpr (PPW == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(xg + j * 8);
        xr[0] = v.x; xr[1] = v.y;
      } else {
#pragma unroll
        for (int q = 0; q < PPW / 4; ++q) {
          const u32x4 v = reinterpret_cast<const u32x4*>(xg + j * PPW * 4)[q];
          xr[4 * q] = v.x; xr[4 * q + 1] = v.y; xr[4 * q + 2] = v.z; xr[4 * q + 3] = v.w;
        }
      }
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const u32x4 v = bf.w[u][j >> 2];
        const uint32_t word = (j & 3) == 0 ? v.x : (j & 3) == 1 ? v.y : (j & 3) == 2 ? v.z : v.w;
        uint32_t h[PPW];
        unpack_word<BITS>(word, h);
#pragma unroll
        for (int p = 0; p < PPW; ++p) {
          if constexpr (GS == 32) {
            // words 0 .. WPG/2-1 hold the first 32-code scale group
            if (j < WPG / 2) a0[u] = j == 0 && p == 0 ? dot2_first(h[p], xr[p]) : dot2(h[p], xr[p], a0[u]);
            else             a1[u] = j == WPG / 2 && p == 0 ? dot2_first(h[p], xr[p]) : dot2(h[p], xr[p], a1[u]);
          } else {
            if ((p & 1) == 0) a0[u] = j == 0 && p == 0 ? dot2_first(h[p], xr[p]) : dot2(h[p], xr[p], a0[u]);
            else              a1[u] = j == 0 && p == 1 ? dot2_first(h[p], xr[p]) : dot2(h[p], xr[p], a1[u]);
          }
        }
      }
    }
    }
    if constexpr (SPLIT && !F::F16W) {
      // folded above
    } else if constexpr (F::F16W) {
#pragma unroll
      for (int u = 0; u < UR; ++u) acc[u] += a0[u] + a1[u];
    } else if constexpr (GS == 32) {
      const float4 c = reinterpret_cast<const float4*>(cx)[g];  // C_lo, X_lo, C_hi, X_hi
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const float s0 = f16_bits_to_f32(bf.s[u][0]), b0 = f16_bits_to_f32(bf.b[u][0]);
        const float s1 = f16_bits_to_f32(bf.s[u][1]), b1 = f16_bits_to_f32(bf.b[u][1]);
        acc[u] = fmaf(s0, a0[u] - c.x, fmaf(b0, c.y, fmaf(s1, a1[u] - c.z, fmaf(b1, c.w, acc[u]))));
      }
    } else {
      const float2 c = reinterpret_cast<const float2*>(cx)[g];
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const float s = f16_bits_to_f32(bf.s[u][0]);
        const float b = f16_bits_to_f32(bf.b[u][0]);
        acc[u] = fmaf(s, (a0[u] + a1[u]) - c.x, fmaf(b, c.y, acc[u]));
      }
    }
    if (++ct == tcount) {
      if constexpr (WK == 1) {
        // end of a pass: reduce over the row's lanes and store
        if constexpr (LPR == 16 && UR <= 4) {
          constexpr int kHold = 16 / UR;  // lanes that end with one row's total
          const float v = row_sum16<UR>(acc, lr);
          const int r = lane_row + cp * Cfg::ROWS + (lr / kHold) * Cfg::RPW;
          if (lr % kHold == 0 && r < row_end) Y[r] = v;
#pragma unroll
          for (int u = 0; u < UR; ++u) acc[u] = 0.0f;
        } else {
#pragma unroll
          for (int u = 0; u < UR; ++u) {
            float v = acc[u];
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m);
            const int r = lane_row + cp * Cfg::ROWS + u * Cfg::RPW;
            if (lr == 0 && r < row_end) Y[r] = v;
            acc[u] = 0.0f;
          }
        }
      }
      ct = 0;
      ++cp;
    }
  };

  // The first step's loads are issued unconditionally (a load under a
  // branch makes the compiler wait for every outstanding load at the join),
  // after the activation loads, so the staging below waits for x only.
  Buf b0, b1;
  const gptr<uint16_t> X = to_global(P.x);
  // A wave whose 64 quarter groups of the first staging round all lie past
  // the end loads and pairs nothing (a wave-uniform branch).  At k = 1024
  // only the first wave has quarters; the other three would otherwise issue
  // the whole pairing and (C, X) sequence for nothing, which the 2- and
  // 3-bit kernels, bound by instruction issue, pay for.
  const bool stager = (int)(threadIdx.x & ~63u) < 4 * groups;
  XStage<BITS> xs;
  if (stager) stage_x_load<BITS>(X, groups, xs);
  issue(b0);
  stage_x_store<BITS, GS>(X, groups, xs, xp, cx, stager);
  __syncthreads();

  for (int st = 0; st < nsteps; st += 2) {
    if (st + 1 < nsteps) issue(b1);
    consume(b0);
    if (st + 1 < nsteps) {
      if (st + 2 < nsteps) issue(b0);
      consume(b1);
    }
  }

  if constexpr (WK > 1) {
    // one pass only (the host guarantees it): reduce lanes, then waves in LDS
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      float v = acc[u];
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m);
      if (lr == 0) red[((wr * UR + u) * Cfg::RPW + slot) * WK + wk] = v;
    }
    __syncthreads();
    if (wk == 0 && lr == 0) {
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const float* rr = red + ((wr * UR + u) * Cfg::RPW + slot) * WK;
        float v = rr[0];
#pragma unroll
        for (int i = 1; i < WK; ++i) v += rr[i];
        const int r = lane_row + u * Cfg::RPW;
        if (r < row_end) Y[r] = v;
      }
    }
  }
}

template <int BITS, int LPR, int UR, int WK, int GS>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(4))) void qgemv_kernel(GemvProblem P, int rows_per_block) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  gemv_block<BITS, LPR, UR, WK, GS>(P, blockIdx.x * rows_per_block, rows_per_block, smem);
}

template <int BITS, int LPR, int UR, int GS>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(4))) void qgemv_batched_kernel(const GemvBlock* __restrict__ blocks) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const GemvBlock blk = blocks[blockIdx.x];
  gemv_block<BITS, LPR, UR, 1, GS>(blk.p, blk.row0, blk.nrows, smem);
}

// ------------------------------------------------------------------ host --

// Rows in flight per lane: fewer for the wider formats (register budget).
constexpr int gemv_ur(int bits) { return bits == 16 ? 1 : bits >= 5 ? 2 : 4; }

int gemv_row_unroll(int bits) { return gemv_ur(bits); }

int gemv_rows_per_pass(int lpr, int ur, int wk) { return (kGemvWaves / wk) * ur * (64 / lpr); }

int gemv_lanes_for_groups(int groups) {
  int lpr = 16;
  while (lpr > 1 && groups % lpr != 0) lpr >>= 1;
  return lpr;
}

GemvGeom gemv_choose(int n, int k, int bits) {
  const int groups = k / 64;
  GemvGeom g;
  g.lanes_per_row = gemv_lanes_for_groups(groups);
  const int T = groups / g.lanes_per_row;
  const int target = 1024;  // workgroups wanted to fill 256 CUs several times over
  g.row_unroll = gemv_row_unroll(bits);
  g.wave_ksplit = 1;
  auto blocks = [&](int ur, int wk) {
    const int r = gemv_rows_per_pass(g.lanes_per_row, ur, wk);
    return (n + r - 1) / r;
  };
  if (blocks(g.row_unroll, 1) < target) g.row_unroll = 1;
  if (blocks(g.row_unroll, 1) < target && T >= 4) g.wave_ksplit = 4;
  g.rows_per_pass = gemv_rows_per_pass(g.lanes_per_row, g.row_unroll, g.wave_ksplit);
  g.passes = 1;  // short workgroups balance best (see qmm_qgemv_batched_plan)
  return g;
}

size_t gemv_lds_bytes(int max_groups, const GemvGeom& g) {
  // per 64-code unit: paired x, and (C, X) once or (for groups of 32) twice
  size_t bytes = (size_t)max_groups * (kXStride + sizeof(float4));
  if (g.wave_ksplit > 1) bytes += (size_t)g.rows_per_pass * g.wave_ksplit * sizeof(float);
  return bytes;
}

template <int BITS, int LPR, int UR, int WK, int GS>
static hipError_t launch_one(const GemvProblem& p, const GemvGeom& g, hipStream_t st, size_t lds) {
  const int rows = GemvCfg<BITS, LPR, UR, WK>::ROWS * g.passes;
  const unsigned grid = (unsigned)((p.n + rows - 1) / rows);
  hipLaunchKernelGGL((qgemv_kernel<BITS, LPR, UR, WK, GS>), dim3(grid), dim3(kGemvThreads), lds, st, p,
                     rows);
  return hipGetLastError();
}

template <int BITS, int LPR, int GS>
static hipError_t launch_lpr(const GemvProblem& p, const GemvGeom& g, hipStream_t st, size_t lds) {
  constexpr int URB = gemv_ur(BITS);
  if (g.row_unroll == URB && g.wave_ksplit == 1) return launch_one<BITS, LPR, URB, 1, GS>(p, g, st, lds);
  if (g.row_unroll == 1 && g.wave_ksplit == 1) return launch_one<BITS, LPR, 1, 1, GS>(p, g, st, lds);
  if (g.row_unroll == 1 && g.wave_ksplit == 4) return launch_one<BITS, LPR, 1, 4, GS>(p, g, st, lds);
  return hipErrorInvalidValue;
}

template <int BITS, int GS>
static hipError_t launch_bits(const GemvProblem& p, const GemvGeom& g, hipStream_t st) {
  const size_t lds = gemv_lds_bytes(p.k / 64, g);
  switch (g.lanes_per_row) {
    case 1: return launch_lpr<BITS, 1, GS>(p, g, st, lds);
    case 2: return launch_lpr<BITS, 2, GS>(p, g, st, lds);
    case 4: return launch_lpr<BITS, 4, GS>(p, g, st, lds);
    case 8: return launch_lpr<BITS, 8, GS>(p, g, st, lds);
    case 16: return launch_lpr<BITS, 16, GS>(p, g, st, lds);
    default: return hipErrorInvalidValue;
  }
}

template <int GS>
static hipError_t launch_gs(const GemvProblem& p, int bits, const GemvGeom& g, hipStream_t st) {
  switch (bits) {
    case 2: return launch_bits<2, GS>(p, g, st);
    case 3: return launch_bits<3, GS>(p, g, st);
    case 4: return launch_bits<4, GS>(p, g, st);
    case 5: return launch_bits<5, GS>(p, g, st);
    case 6: return launch_bits<6, GS>(p, g, st);
    case 8: return launch_bits<8, GS>(p, g, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_qgemv(const GemvProblem& p, int bits, int group_size, const GemvGeom& g,
                        hipStream_t st) {
  if (bits == 16) return launch_bits<16, 64>(p, g, st);  // no scale groups
  switch (group_size) {
    case 32: return launch_gs<32>(p, bits, g, st);
    case 64: return launch_gs<64>(p, bits, g, st);
    case 128: return launch_gs<128>(p, bits, g, st);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS, int LPR, int GS>
static hipError_t launch_batched_one(const GemvBlock* blocks, int num_blocks, size_t lds,
                                     hipStream_t st) {
  constexpr int URB = gemv_ur(BITS);
  hipLaunchKernelGGL((qgemv_batched_kernel<BITS, LPR, URB, GS>), dim3(num_blocks), dim3(kGemvThreads),
                     lds, st, blocks);
  return hipGetLastError();
}

template <int BITS, int GS>
static hipError_t launch_batched_bits(const GemvBlock* blocks, int num_blocks, int lpr,
                                      size_t lds, hipStream_t st) {
  switch (lpr) {
    case 1: return launch_batched_one<BITS, 1, GS>(blocks, num_blocks, lds, st);
    case 2: return launch_batched_one<BITS, 2, GS>(blocks, num_blocks, lds, st);
    case 4: return launch_batched_one<BITS, 4, GS>(blocks, num_blocks, lds, st);
    case 8: return launch_batched_one<BITS, 8, GS>(blocks, num_blocks, lds, st);
    case 16: return launch_batched_one<BITS, 16, GS>(blocks, num_blocks, lds, st);
    default: return hipErrorInvalidValue;
  }
}

template <int GS>
static hipError_t launch_batched_gs(const GemvBlock* blocks, int num_blocks, int bits, int lpr,
                                    size_t lds, hipStream_t st) {
  switch (bits) {
    case 2: return launch_batched_bits<2, GS>(blocks, num_blocks, lpr, lds, st);
    case 3: return launch_batched_bits<3, GS>(blocks, num_blocks, lpr, lds, st);
    case 4: return launch_batched_bits<4, GS>(blocks, num_blocks, lpr, lds, st);
    case 5: return launch_batched_bits<5, GS>(blocks, num_blocks, lpr, lds, st);
    case 6: return launch_batched_bits<6, GS>(blocks, num_blocks, lpr, lds, st);
    case 8: return launch_batched_bits<8, GS>(blocks, num_blocks, lpr, lds, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_qgemv_batched(const GemvBlock* blocks, int num_blocks, int bits, int group_size,
                                int lanes_per_row, int max_groups, hipStream_t st) {
  GemvGeom g{lanes_per_row, gemv_row_unroll(bits), 1,
             gemv_rows_per_pass(lanes_per_row, gemv_row_unroll(bits), 1), 1};
  const size_t lds = gemv_lds_bytes(max_groups, g);
  if (bits == 16) return launch_batched_bits<16, 64>(blocks, num_blocks, lanes_per_row, lds, st);
  switch (group_size) {
    case 32: return launch_batched_gs<32>(blocks, num_blocks, bits, lanes_per_row, lds, st);
    case 64: return launch_batched_gs<64>(blocks, num_blocks, bits, lanes_per_row, lds, st);
    case 128: return launch_batched_gs<128>(blocks, num_blocks, bits, lanes_per_row, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmm
