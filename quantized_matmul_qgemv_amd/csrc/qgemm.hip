// Prefill GEMM over group-quantized weights: y[m, n] = sum_k x[m, k] W_hat[n, k]
// (BaseRT, native-Metal LLM inference on Apple Silicon, §3.4: tile
// geometry chosen per sequence-length range).  The tile core is in
// qgemm_core.h; this file picks the tile and maps workgroups to tiles.
#include "qgemm_core.h"
#include "qmm_internal.h"

namespace qmm {

template <int BITS, int BM, int NB>
__global__ __launch_bounds__(kGemmThreads) void qgemm_kernel(GemmArgs a, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BM * kAStrideHalves];
  constexpr int BN = 4 * NB * 32;
  // Consecutive workgroups take consecutive column tiles of the same rows
  // tile; column tiles that share weights are then spread over XCDs only
  // across row tiles.
  const int tile = blockIdx.x;
  const int tn = tile % n_tiles;
  const int tm = tile / n_tiles;
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int m = a.m;
  auto a_row = [&](int i) { const int r = m0 + i; return r < m ? r : m - 1; };
  auto c_row = [&](int i) { const int r = m0 + i; return r < m ? r : -1; };
  gemm_tile<BITS, BM, NB>(ARows{a.x, a.k}, a_row, c_row, a.w, a.s, a.b, a.y, a.n, n0, a.n, lds);
}

template <int BITS, int BM, int NB>
static hipError_t launch_tile(const GemmArgs& a, hipStream_t st) {
  constexpr int BN = 4 * NB * 32;
  const int n_tiles = (a.n + BN - 1) / BN;
  const int m_tiles = (a.m + BM - 1) / BM;
  hipLaunchKernelGGL((qgemm_kernel<BITS, BM, NB>), dim3(n_tiles * m_tiles), dim3(kGemmThreads), 0,
                     st, a, n_tiles);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_bits(const GemmArgs& a, hipStream_t st) {
  // Tile choice: the largest row tile that the rows fill, then the wider
  // column tile only when it still leaves at least two workgroups per CU.
  const int cus = 256;
  if (a.m <= 32) return launch_tile<BITS, 32, 1>(a, st);
  if (a.m <= 64) return launch_tile<BITS, 64, 1>(a, st);
  const long tiles_wide = (long)((a.n + 255) / 256) * ((a.m + 127) / 128);
  if (tiles_wide >= 2 * cus) return launch_tile<BITS, 128, 2>(a, st);
  return launch_tile<BITS, 128, 1>(a, st);
}

hipError_t launch_qgemm(const GemmArgs& a, int bits, hipStream_t st) {
  switch (bits) {
    case 2: return launch_bits<2>(a, st);
    case 4: return launch_bits<4>(a, st);
    case 8: return launch_bits<8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmm
