// Prefill GEMM over group-quantized weights: y[m, n] = sum_k x[m, k] W_hat[n, k]
// (BaseRT, native-Metal LLM inference on Apple Silicon, §3.4: tile
// geometry chosen per sequence-length range).  The tile cores are in
// qgemm_core.h and qgemm_wide.h; the tile shape and k-split count come from
// the planner shared with the batched GEMM (gemm_choose in
// qgemm_batched.hip); this file maps workgroups to tiles and sums split-k
// partials.
//
// Workgroup -> tile mapping.  Workgroups are dealt round-robin to the 8
// XCDs (each with its own L2).  Tiles that share weight columns (same
// column tile and k split, different row tiles) are numbered consecutively
// and each XCD gets a contiguous range of tile numbers, so a weight column
// tile is read from HBM into one L2 and reused there by all its row tiles.
//
// Split-k.  With S splits, workgroup (tile, split) accumulates the groups
// [split*G/S, (split+1)*G/S) and writes its fp32 partial tile to the
// workspace; qgemm_reduce_kernel then sums the S partials of every output
// in split order, so the result does not depend on scheduling.
#include "qgemm_core.h"
#include "qgemm_wide.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int kXcds = 8;

struct GemmGrid {
  int n_tiles, m_tiles, splits, gps_split;  // groups per split
  int xcd_remap;
  long stride;                               // floats between partial tiles of two splits
};

template <int BITS, int BM, int NB, bool SBQ>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2))) void qgemm_kernel(GemmArgs a, GemmGrid gr, float* partial) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BM * kAStride];
  constexpr int BN = 4 * NB * 32;
  const int total = gr.n_tiles * gr.m_tiles * gr.splits;
  int t = blockIdx.x;
  if (gr.xcd_remap) t = (t % kXcds) * (total / kXcds) + t / kXcds;
  const int tm = t % gr.m_tiles;
  const int rest = t / gr.m_tiles;
  const int split = rest % gr.splits;
  const int tn = rest / gr.splits;
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int m = a.m;
  auto a_row = [&](int i) { const int r = m0 + i; return r < m ? r : m - 1; };
  auto c_row = [&](int i) { const int r = m0 + i; return r < m ? r : -1; };
  float* out = gr.splits == 1 ? a.y : partial + (size_t)split * gr.stride;
  const int g0 = split * gr.gps_split;
  const int g1 = g0 + gr.gps_split;
  gemm_tile<BITS, BM, NB, SBQ>(ARows{a.x, a.k}, a_row, c_row, a.w, a.s, a.b, out + n0, a.n, n0,
                               a.n, g0, g1, lds, a.group_size, nullptr, nullptr, nullptr, nullptr,
                               a.wtiled, a.stiled);
}

// 256 x 256 tiles, one workgroup per CU (qgemm_wide.h); same tile order as
// qgemm_kernel.
template <int BITS, bool SBQ>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(1))) void qgemm_wide_kernel(GemmArgs a, GemmGrid gr, float* partial) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kWideLdsHalves];
  constexpr int BM = kWideBM;
  constexpr int BN = 256;
  const int total = gr.n_tiles * gr.m_tiles * gr.splits;
  int t = blockIdx.x;
  if (gr.xcd_remap) t = (t % kXcds) * (total / kXcds) + t / kXcds;
  const int tm = t % gr.m_tiles;
  const int rest = t / gr.m_tiles;
  const int split = rest % gr.splits;
  const int tn = rest / gr.splits;
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int m = a.m;
  auto a_row = [&](int i) { const int r = m0 + i; return r < m ? r : m - 1; };
  auto c_row = [&](int i) { const int r = m0 + i; return r < m ? r : -1; };
  float* out = gr.splits == 1 ? a.y : partial + (size_t)split * gr.stride;
  const int g0 = split * gr.gps_split;
  const int g1 = g0 + gr.gps_split;
  gemm_tile_wide<BITS, SBQ>(ARows{a.x, a.k}, a_row, c_row, a.w, a.s, a.b, out + n0, a.n, n0, a.n,
                            g0, g1, lds, a.group_size, a.wtiled, a.stiled);
}

// y[i] = sum over splits of partial[split * stride + i], in split order.
// S > 0: the split count as a template argument, so that all S loads are
// issued before the first addition (split order kept); S = 0: run-time count.
template <int S>
__global__ __launch_bounds__(256) void qgemm_reduce_kernel(const float* __restrict__ partial,
                                                           float* __restrict__ y, long count,
                                                           long stride, int splits) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float acc;
  if constexpr (S > 0) {
    float v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = partial[(size_t)s * stride + i];
    acc = v[0];
#pragma unroll
    for (int s = 1; s < S; ++s) acc += v[s];
  } else {
    acc = partial[i];
    for (int s = 1; s < splits; ++s) acc += partial[(size_t)s * stride + i];
  }
  y[i] = acc;
}

static void launch_reduce(const float* ws, float* y, long count, long stride, int splits, hipStream_t st) {
  const dim3 grid((unsigned)((count + 255) / 256));
  switch (splits) {
#define QMM_REDUCE_CASE(S) \
    case S: hipLaunchKernelGGL(qgemm_reduce_kernel<S>, grid, dim3(256), 0, st, ws, y, count, stride, S); break;
    QMM_REDUCE_CASE(2) QMM_REDUCE_CASE(3) QMM_REDUCE_CASE(4) QMM_REDUCE_CASE(5) QMM_REDUCE_CASE(6)
    QMM_REDUCE_CASE(8) QMM_REDUCE_CASE(10) QMM_REDUCE_CASE(12) QMM_REDUCE_CASE(16)
#undef QMM_REDUCE_CASE
    default: hipLaunchKernelGGL(qgemm_reduce_kernel<0>, grid, dim3(256), 0, st, ws, y, count, stride, splits);
  }
}

// Partial tiles of one split are `partial_stride` floats apart (a multiple
// of 64 floats, so every split starts 256-byte aligned).
static long partial_stride(int m, int n) { return ((long)m * n + 63) / 64 * 64; }

// ------------------------------------------------------------------ host --

// Tile / split choice for one GEMM.
struct GemmPlan {
  int bm, nb, splits;
};

static int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

static GemmPlan gemm_plan(int m, int n, int k, int bits) {
  GemmPlan p;
  gemm_choose(m, n, k, bits, &p.bm, &p.nb, &p.splits);
  return p;
}

size_t gemm_workspace_bytes(int m, int n, int k, int bits) {
  const GemmPlan p = gemm_plan(m, n, k, bits);
  return p.splits > 1 ? (size_t)p.splits * partial_stride(m, n) * sizeof(float) : 0;
}

template <int BITS, int BM, int NB, bool SBQ>
static hipError_t launch_tile(const GemmArgs& a, const GemmPlan& p, float* ws, hipStream_t st) {
  constexpr int BN = 4 * NB * 32;
  GemmGrid gr;
  gr.n_tiles = ceil_div(a.n, BN);
  gr.m_tiles = ceil_div(a.m, BM);
  gr.splits = p.splits;
  gr.gps_split = (a.k / 64) / p.splits;
  const int total = gr.n_tiles * gr.m_tiles * gr.splits;
  gr.xcd_remap = total % kXcds == 0 ? 1 : 0;
  gr.stride = partial_stride(a.m, a.n);
  hipLaunchKernelGGL((qgemm_kernel<BITS, BM, NB, SBQ>), dim3(total), dim3(kGemmThreads), 0, st, a,
                     gr, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const long count = (long)a.m * a.n;
  launch_reduce(ws, a.y, count, gr.stride, p.splits, st);
  return hipGetLastError();
}

template <int BITS, bool SBQ>
static hipError_t launch_wide(const GemmArgs& a, const GemmPlan& p, float* ws, hipStream_t st) {
  GemmGrid gr;
  gr.n_tiles = ceil_div(a.n, 256);
  gr.m_tiles = ceil_div(a.m, kWideBM);
  gr.splits = p.splits;
  gr.gps_split = (a.k / 64) / p.splits;
  const int total = gr.n_tiles * gr.m_tiles * gr.splits;
  gr.xcd_remap = total % kXcds == 0 ? 1 : 0;
  gr.stride = partial_stride(a.m, a.n);
  hipLaunchKernelGGL((qgemm_wide_kernel<BITS, SBQ>), dim3(total), dim3(kGemmThreads), 0, st, a, gr, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const long count = (long)a.m * a.n;
  launch_reduce(ws, a.y, count, gr.stride, p.splits, st);
  return hipGetLastError();
}

template <int BITS, int BM>
static hipError_t launch_bm(const GemmArgs& a, const GemmPlan& p, float* ws, hipStream_t st) {
  // quad scale loads (8 bytes per column): groups of 64, whole quads per
  // split, and 8-byte aligned scale and bias arrays
  const bool sbq = ((a.k / 64) / p.splits) % 4 == 0 && a.group_size == 64 &&
                   ((uintptr_t)a.s & 7) == 0 && ((uintptr_t)a.b & 7) == 0;
  if (p.nb == 2)
    return sbq ? launch_tile<BITS, BM, 2, true>(a, p, ws, st) : launch_tile<BITS, BM, 2, false>(a, p, ws, st);
  return sbq ? launch_tile<BITS, BM, 1, true>(a, p, ws, st) : launch_tile<BITS, BM, 1, false>(a, p, ws, st);
}

template <int BITS>
static hipError_t launch_bits(const GemmArgs& a, const GemmPlan& p, float* ws, hipStream_t st) {
  if constexpr (BITS == 16) {  // fp16 weights: nb = 1 tiles, no scales (see gemm_choose)
    switch (p.bm) {
      case 32: return launch_tile<16, 32, 1, false>(a, p, ws, st);
      case 64: return launch_tile<16, 64, 1, false>(a, p, ws, st);
      default: return launch_tile<16, 128, 1, false>(a, p, ws, st);
    }
  } else {
    switch (p.bm) {
      case 32: return launch_bm<BITS, 32>(a, p, ws, st);
      case 64: return launch_bm<BITS, 64>(a, p, ws, st);
      case 256:
        return ((a.k / 64) / p.splits) % 4 == 0 && a.group_size == 64 ? launch_wide<BITS, true>(a, p, ws, st)
                                                : launch_wide<BITS, false>(a, p, ws, st);
      default: return launch_bm<BITS, 128>(a, p, ws, st);
    }
  }
}

hipError_t launch_qgemm(const GemmArgs& a, int bits, void* workspace, hipStream_t st) {
  const GemmPlan p = gemm_plan(a.m, a.n, a.k, bits);
  float* ws = reinterpret_cast<float*>(workspace);
  switch (bits) {
    case 2: return launch_bits<2>(a, p, ws, st);
    case 3: return launch_bits<3>(a, p, ws, st);
    case 4: return launch_bits<4>(a, p, ws, st);
    case 5: return launch_bits<5>(a, p, ws, st);
    case 6: return launch_bits<6>(a, p, ws, st);
    case 8: return launch_bits<8>(a, p, ws, st);
    case 16: return launch_bits<16>(a, p, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmm
