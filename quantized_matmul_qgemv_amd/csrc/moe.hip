// Mixture-of-experts grouped GEMM (BaseRT, native-Metal LLM inference on
// Apple Silicon: abstract and Fig. 1, MoE prefill on Qwen3-30B-A3B).  The
// pages give no mechanism; this one is token-to-expert bucketing followed
// by one tile schedule per expert:
//
//   1. bucket (one workgroup, all in LDS): histogram of expert ids,
//      exclusive scans (wave shuffles, then across waves) of the per-expert
//      pair counts and of the per-expert row-tile counts, scatter of pair
//      indices into per-expert buckets, and a flat list of row tiles
//      {expert, first bucket slot, rows}.
//   2. grouped GEMM: the grid is an upper bound on (row tiles) x (column
//      tiles); each workgroup reads its row tile from the list (extra
//      workgroups exit at once), gathers its A rows through the bucket,
//      multiplies them by its expert's weights with the GEMM tile core and
//      scatters the output rows back to pair order.
//
// The order of pairs inside a bucket depends on atomic scheduling, but each
// output row is computed on its own (the matrix-core accumulation order
// over k does not depend on the other rows of the tile), so results are
// bit-identical from run to run.
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "qgemm_core.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int kBucketThreads = 1024;
constexpr int kMaxExperts = 1024;

struct MoeTile {
  int32_t expert;  // -1: the pairs whose expert id lies outside [0, E)
  int32_t start;   // first slot in the sorted pair list
  int32_t rows;
};

// Workspace layout (int32 units): a header of kPlanHeaderInts words
//   [0] row tiles in the list   [1] row tile (rows)   [2] pairs   [3] experts
//   [4] pairs whose expert id is outside [0, E) (their output rows are NaN)
//   [5..7] zero
// then the sorted pairs (P words) and the tile list (3 words per tile).  The
// same image is the routing plan that one bucketing pass builds for several
// grouped GEMMs on the same expert ids.  Pairs with an out-of-range id sit
// after every valid bucket and get row tiles of their own (expert -1), so
// the bound on row tiles counts E + 1 buckets.
constexpr int kPlanHeaderInts = 8;
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static int max_row_tiles(int pairs, int experts, int bm) {
  const long by_pairs = (long)(pairs + bm - 1) / bm + experts + 1;
  return by_pairs < pairs ? (int)by_pairs : (pairs > 0 ? pairs : 1);
}

static int route_chunks(int pairs, int experts, int* chunk);

size_t grouped_workspace_bytes(int t, int top_k, int e, int n) {
  (void)n;
  const long pairs = (long)t * top_k;
  const long tiles = max_row_tiles((int)pairs, e, 32);
  int chunk;
  const long counts = (long)route_chunks((int)pairs, e, &chunk) * (e + 1);
  return align_up((size_t)(kPlanHeaderInts + pairs + 3 * tiles + counts) * sizeof(int32_t), 256);
}

// Inclusive sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Bucketing runs as two launches over chunks of the pair list, so that the
// LDS atomics that count and place the pairs are spread over many CUs (one
// workgroup doing all of them was bound by same-address conflicts on its one
// LDS: about 20 us for 16384 pairs).
//   count:   workgroup c histograms the expert ids of pairs
//            [c * chunk, (c + 1) * chunk) into counts[c][0 .. E] (slot E:
//            out-of-range ids).
//   scatter: every workgroup sums the count columns (all chunks, and the
//            chunks before its own), scans them over the experts into bucket
//            starts, and places its own chunk's pairs from there; workgroup
//            0 also writes the tile list and the header.
// The counts (chunks x (E + 1) words) follow the tile list in the workspace.
// Up to kRouteSingleMax pairs there is one chunk and one launch.
constexpr int kCountThreads = 256;
constexpr int kRouteChunkMin = 256;     // pairs per chunk at least
constexpr int kRouteMaxChunks = 64;
constexpr int kRouteCountWords = 32768; // chunks x (E + 1) at most
// Up to this many pairs the scatter launch histograms all of them itself
// and the count launch is skipped: two launches cost about 10 us whatever
// the size, one workgroup doing every atomic about 7 us at 4096 pairs.
constexpr int kRouteSingleMax = 4096;

static int route_chunks(int pairs, int experts, int* chunk) {
  if (pairs <= kRouteSingleMax) {  // one chunk: the scatter launch counts it itself
    *chunk = pairs > 0 ? pairs : 1;
    return 1;
  }
  int g = kRouteCountWords / (experts + 1);
  g = g < 1 ? 1 : (g > kRouteMaxChunks ? kRouteMaxChunks : g);
  int c = (pairs + g - 1) / g;
  c = c < kRouteChunkMin ? kRouteChunkMin : c;
  *chunk = c;
  return pairs > 0 ? (pairs + c - 1) / c : 1;
}

static int32_t* route_counts(int32_t* ws, int pairs, int experts) {
  return ws + kPlanHeaderInts + pairs + 3 * (size_t)max_row_tiles(pairs, experts, 32);
}

__global__ __launch_bounds__(kCountThreads) void moe_count_kernel(const int32_t* __restrict__ ids, int pairs,
                                                                   int experts, int chunk,
                                                                   int32_t* __restrict__ counts) {
  __shared__ int32_t h[kMaxExperts + 1];
  for (int i = threadIdx.x; i <= experts; i += kCountThreads) h[i] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * chunk;
  const int p1 = p0 + chunk < pairs ? p0 + chunk : pairs;
  for (int p = p0 + threadIdx.x; p < p1; p += kCountThreads) {
    const int e = ids[p];
    atomicAdd(&h[e >= 0 && e < experts ? e : experts], 1);
  }
  __syncthreads();
  int32_t* row = counts + (size_t)blockIdx.x * (experts + 1);
  for (int i = threadIdx.x; i <= experts; i += kCountThreads) row[i] = h[i];
}

__global__ __launch_bounds__(kBucketThreads) void moe_scatter_kernel(
    const int32_t* __restrict__ ids, int pairs, int experts, int bm, int chunk, int chunks,
    const int32_t* __restrict__ counts, int32_t* __restrict__ ws) {
  static_assert(kBucketThreads == kMaxExperts, "one thread per expert slot");
  constexpr int kWaves = kBucketThreads / 64;
  __shared__ int32_t cursor[kMaxExperts];
  __shared__ int32_t total[kMaxExperts + 1];   // per slot: pairs in all chunks
  __shared__ int32_t earlier[kMaxExperts + 1]; // per slot: pairs in the chunks before this one
  __shared__ int32_t wtot[2][kWaves];
  __shared__ int32_t bad_cursor;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int me = blockIdx.x;
  int32_t* sorted = ws + kPlanHeaderInts;
  MoeTile* tiles = reinterpret_cast<MoeTile*>(ws + kPlanHeaderInts + pairs);
  const int stride = experts + 1;

  // column sums over the chunks x (E + 1) counts, all threads taking words
  // in turn: a batch of independent loads per thread, then LDS additions;
  // with no counts (a single chunk) the histogram of the ids themselves
  for (int i = tid; i <= experts; i += kBucketThreads) total[i] = earlier[i] = 0;
  __syncthreads();
  if (counts == nullptr) {
    for (int p = tid; p < pairs; p += kBucketThreads) {
      const int e = ids[p];
      atomicAdd(&total[e >= 0 && e < experts ? e : experts], 1);
    }
  }
  const int ncounts = counts == nullptr ? 0 : chunks * stride;
  constexpr int kSumLoads = 16;
  for (int base = 0; base < ncounts; base += kBucketThreads * kSumLoads) {
    int v[kSumLoads];
#pragma unroll
    for (int j = 0; j < kSumLoads; ++j) {
      const int i = base + j * kBucketThreads + tid;
      v[j] = i < ncounts ? counts[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kSumLoads; ++j) {
      if (v[j] == 0) continue;
      const int i = base + j * kBucketThreads + tid;
      const int w = i / stride;
      const int e = i - w * stride;
      atomicAdd(&total[e], v[j]);
      if (w < me) atomicAdd(&earlier[e], v[j]);
    }
  }
  __syncthreads();
  const int c = tid < experts ? total[tid] : 0;
  const int before = tid < experts ? earlier[tid] : 0;
  const int bad = tid == 0 ? total[experts] : 0;
  // exclusive scans of the pair counts and of the row-tile counts:
  // within each wave by lane shuffles, then over the 16 wave totals
  const int tl = (c + bm - 1) / bm;
  const int ic = wave_inclusive_sum(c);
  const int it = wave_inclusive_sum(tl);
  if (lane == 63) {
    wtot[0][wave] = ic;
    wtot[1][wave] = it;
  }
  __syncthreads();
  if (wave == 0) {
    const int a0 = lane < kWaves ? wtot[0][lane] : 0;
    const int a1 = lane < kWaves ? wtot[1][lane] : 0;
    const int s0 = wave_inclusive_sum(a0);
    const int s1 = wave_inclusive_sum(a1);
    if (lane < kWaves) {
      wtot[0][lane] = s0 - a0;  // exclusive prefix of the wave totals
      wtot[1][lane] = s1 - a1;
    }
    // the out-of-range pairs follow every valid bucket, with tiles of their own
    const int valid = __shfl(s0, kWaves - 1, 64);
    const int tiles_valid = __shfl(s1, kWaves - 1, 64);
    const int nbad = __shfl(bad, 0, 64);
    if (lane == 0) bad_cursor = valid + earlier[experts];
    if (me == 0 && lane == 0) {
      const int bad_tiles = (nbad + bm - 1) / bm;
      for (int i = 0; i < bad_tiles; ++i)
        tiles[tiles_valid + i] = MoeTile{-1, valid + i * bm, nbad - i * bm < bm ? nbad - i * bm : bm};
      ws[0] = tiles_valid + bad_tiles;
      ws[4] = nbad;
    }
  }
  __syncthreads();
  const int start = wtot[0][wave] + ic - c;
  const int tstart = wtot[1][wave] + it - tl;
  cursor[tid] = start + before;
  __syncthreads();
  // place this chunk's pairs in their expert's bucket
  const int p0 = me * chunk;
  const int p1 = p0 + chunk < pairs ? p0 + chunk : pairs;
  for (int p = p0 + tid; p < p1; p += kBucketThreads) {
    const int e = ids[p];
    sorted[e >= 0 && e < experts ? atomicAdd(&cursor[e], 1) : atomicAdd(&bad_cursor, 1)] = p;
  }
  if (me == 0) {
    if (tid < experts) {
      for (int i = 0; i < tl; ++i) {
        const int rows = c - i * bm < bm ? c - i * bm : bm;
        tiles[tstart + i] = MoeTile{tid, start + i * bm, rows};
      }
    }
    if (tid == 0) {  // what the plan was built for (checked by every grouped kernel)
      ws[1] = bm;
      ws[2] = pairs;
      ws[3] = experts;
      ws[5] = 0;
      ws[6] = 0;
      ws[7] = 0;
    }
  }
}

static hipError_t launch_bucket(const int32_t* ids, int pairs, int experts, int bm, int32_t* ws,
                                hipStream_t st) {
  int chunk;
  const int chunks = route_chunks(pairs, experts, &chunk);
  int32_t* counts = nullptr;
  if (chunks > 1) {
    counts = route_counts(ws, pairs, experts);
    hipLaunchKernelGGL(moe_count_kernel, dim3(chunks), dim3(kCountThreads), 0, st, ids, pairs, experts, chunk,
                       counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(chunks), dim3(kBucketThreads), 0, st, ids, pairs, experts, bm,
                     chunk, chunks, counts, ws);
  return hipGetLastError();
}

// Output of a grouped launch that cannot be computed: a plan built for
// another row tile, pair count or expert count.  The whole output
// (rows x cols elements, row stride ld) is filled with NaN by the launch's
// workgroups together, so the failure shows in every result.
template <typename T>
__device__ void fill_nan_all(T* out, long rows, int cols, int ld, T nan) {
  const long total = rows * cols;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride)
    out[(i / cols) * ld + i % cols] = nan;
}

// Rows of the pairs of an out-of-range row tile (expert -1): NaN in the
// tile's columns [c0, c0 + bn) (bounded by n).
template <typename T>
__device__ void fill_nan_rows(T* out, const int32_t* sorted, const MoeTile& mt, int c0, int bn, int n,
                              T nan) {
  const int cols = n - c0 < bn ? n - c0 : bn;
  for (int i = threadIdx.x; i < mt.rows * cols; i += blockDim.x) {
    const long row = sorted[mt.start + i / cols];
    out[row * n + c0 + i % cols] = nan;
  }
}

// Workgroup -> (row tile, column tile).  Workgroups are dealt round-robin
// to the 8 XCDs (workgroup b runs on XCD b % 8), each with its own L2.  All
// column tiles of one row tile gather the same A rows (the expert's tokens),
// and consecutive row tiles of the list belong mostly to one expert and read
// the same weights; so runs of kMoeRun consecutive row tiles, with all their
// column tiles, are placed on one XCD, next to each other in its dispatch
// order, and the runs are dealt round-robin across the XCDs:
//   b -> xcd = b % 8, i = b / 8, k = i / n_tiles;
//   row tile = (k / R) * 8R + xcd * R + k % R,  column tile = i % n_tiles
// (R = kMoeRun).  The grid is ceil(row tiles / 8R) * 8R * n_tiles
// workgroups.  Against one row tile per run (R = 1) this halved the bytes
// the grouped GEMM and the fused gate/up fetch at 2048 tokens (443 -> 243 MB
// and 998 -> 493 MB per launch) and took the fused gate/up from 177 to
// 160 us.
constexpr int kMoeXcds = 8;
constexpr int kMoeRun = 8;

__device__ __forceinline__ void moe_tile_of(int n_tiles, int run, int& tile, int& tn) {
  const int xcd = blockIdx.x % kMoeXcds;
  const int i = blockIdx.x / kMoeXcds;
  const int k = i / n_tiles;
  tile = (k / run) * (kMoeXcds * run) + xcd * run + k % run;
  tn = i % n_tiles;
}

static unsigned moe_grid(int m_tiles, int n_tiles, int run) {
  const int per = kMoeXcds * run;
  return (unsigned)((m_tiles + per - 1) / per) * per * n_tiles;
}

// Waves per SIMD the register allocator is held to: two, except for the
// 128-row, 256-column tiles of the 5- to 16-bit formats and the 160-row
// fused gate/up tiles (160 accumulators per lane), which would spill at two
// and keep the whole register file at one.
constexpr int moe_waves(int bits, int bm, int nb) {
  return (nb == 2 && ((bm == 128 && bits >= 5) || bm == 160)) ? 1 : 2;
}

template <int BITS, int BM, int NB, bool SBQ>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(moe_waves(BITS, BM, NB))))
void grouped_kernel(GroupedArgs a, const int32_t* __restrict__ ws, int n_tiles, int run) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BM * kAStride];
  __shared__ int32_t pair_of[BM];
  constexpr int BN = 4 * NB * 32;
  const int pairs = a.t * a.top_k;
  int tile, tn;
  moe_tile_of(n_tiles, run, tile, tn);
  // a routing plan built for another row tile, pair count or expert count
  // is not used: the whole output becomes NaN
  if (ws[1] != BM || ws[2] != pairs || ws[3] != a.e) {
    fill_nan_all(a.y, pairs, a.n, a.n, __builtin_nanf(""));
    return;
  }
  if (tile >= ws[0]) return;
  const MoeTile mt = reinterpret_cast<const MoeTile*>(ws + kPlanHeaderInts + pairs)[tile];
  const int32_t* sorted = ws + kPlanHeaderInts;
  if (mt.expert < 0) {  // pairs with an out-of-range expert id
    fill_nan_rows(a.y, sorted, mt, tn * BN, BN, a.n, __builtin_nanf(""));
    return;
  }
  for (int i = threadIdx.x; i < BM; i += blockDim.x)
    pair_of[i] = sorted[mt.start + (i < mt.rows ? i : mt.rows - 1)];
  __syncthreads();
  const int top_k = a.top_k;
  const int per_pair = a.a_row_per_pair;
  const int rows = mt.rows;
  auto a_row = [&](int i) { const int p = pair_of[i]; return per_pair ? p : p / top_k; };
  auto c_row = [&](int i) { return i < rows ? pair_of[i] : -1; };
  const int groups = a.k >> 6;
  const size_t wstride = (size_t)a.n * groups * Fmt<BITS>::WORDS_PER_GROUP;
  // interleaved scales hold the biases too: twice the halves per expert
  const size_t sstride = (size_t)a.n * (a.k / a.group_size) * (a.stiled ? 2 : 1);
  gemm_tile<BITS, BM, NB, SBQ>(ARows{a.a, a.k}, a_row, c_row, a.w + mt.expert * wstride,
                               a.s + mt.expert * sstride, a.stiled ? nullptr : a.b + mt.expert * sstride,
                               a.y + tn * BN,
                               a.n, tn * BN, a.n, 0, groups, lds, a.group_size, nullptr, nullptr, nullptr,
                               nullptr, a.wtiled, a.stiled);
}

// Fused gate + up with the SwiGLU epilogue: one workgroup computes, for
// its row tile and 128 columns, both products of the token rows with the
// expert's gate and up weights and writes h = silu(gate) * up in fp16 (the
// down projection's input), so neither fp32 product goes to memory.
static void moe_tile(int pairs, int experts, int stiled, int* bm_out, int* nb_out);

struct SwigluArgs {
  const uint32_t* wg;
  const uint16_t* sg;
  const uint16_t* bg;
  const uint32_t* wu;
  const uint16_t* su;
  const uint16_t* bu;
  const uint16_t* x;
  uint16_t* h;
  int t, top_k, e, n, k, group_size;
  int wtiled;  // weights in the tile-interleaved layout (qmm_repack_tiled)
  int stiled;  // scales and biases interleaved (qmm_repack_scales_tiled; sg, su hold both)
};

template <int BITS, int BM, bool SBQ>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(moe_waves(BITS, BM, 2))))
void swiglu_kernel(SwigluArgs a, const int32_t* __restrict__ ws, int n_tiles, int run) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BM * kAStride];
  __shared__ int32_t pair_of[BM];
  const int pairs = a.t * a.top_k;
  int tile, tn;
  moe_tile_of(n_tiles, run, tile, tn);
  const uint16_t nan16 = 0x7E00;  // fp16 quiet NaN
  if (ws[1] != BM || ws[2] != pairs || ws[3] != a.e) {  // foreign plan: h is all NaN
    fill_nan_all(a.h, pairs, a.n, a.n, nan16);
    return;
  }
  if (tile >= ws[0]) return;
  const MoeTile mt = reinterpret_cast<const MoeTile*>(ws + kPlanHeaderInts + pairs)[tile];
  const int32_t* sorted = ws + kPlanHeaderInts;
  if (mt.expert < 0) {  // pairs with an out-of-range expert id
    fill_nan_rows(a.h, sorted, mt, tn * 128, 128, a.n, nan16);
    return;
  }
  for (int i = threadIdx.x; i < BM; i += blockDim.x)
    pair_of[i] = sorted[mt.start + (i < mt.rows ? i : mt.rows - 1)];
  __syncthreads();
  const int top_k = a.top_k;
  const int rows = mt.rows;
  auto a_row = [&](int i) { return pair_of[i] / top_k; };
  auto c_row = [&](int i) { return i < rows ? pair_of[i] : -1; };
  const int groups = a.k >> 6;
  const size_t wstride = (size_t)a.n * groups * Fmt<BITS>::WORDS_PER_GROUP;
  const size_t sstride = (size_t)a.n * (a.k / a.group_size) * (a.stiled ? 2 : 1);
  const size_t eo = (size_t)mt.expert;
  gemm_tile<BITS, BM, 2, SBQ, true>(ARows{a.x, a.k}, a_row, c_row, a.wg + eo * wstride,
                                    a.sg + eo * sstride, a.stiled ? nullptr : a.bg + eo * sstride, nullptr, a.n,
                                    tn * 128, a.n, 0, groups, lds, a.group_size,
                                    a.wu + eo * wstride, a.su + eo * sstride,
                                    a.stiled ? nullptr : a.bu + eo * sstride, a.h + tn * 128, a.wtiled,
                                    a.stiled);
}

template <int BITS, bool SBQ>
static hipError_t launch_swiglu_sbq(const SwigluArgs& a, const int32_t* plan, hipStream_t st) {
  int bm, nb;  // the fused tile is always 128 columns wide
  moe_tile(a.t * a.top_k, a.e, a.stiled, &bm, &nb);
  const int n_tiles = (a.n + 127) / 128;
  const int m_tiles = max_row_tiles(a.t * a.top_k, a.e, bm);
  const int run = kMoeRun;
  const dim3 grid(moe_grid(m_tiles, n_tiles, run));
  if (bm == 32) hipLaunchKernelGGL((swiglu_kernel<BITS, 32, SBQ>), grid, dim3(kGemmThreads), 0, st, a, plan, n_tiles, run);
  else if (bm == 64) hipLaunchKernelGGL((swiglu_kernel<BITS, 64, SBQ>), grid, dim3(kGemmThreads), 0, st, a, plan, n_tiles, run);
  else if (bm == 160) hipLaunchKernelGGL((swiglu_kernel<BITS, 160, SBQ>), grid, dim3(kGemmThreads), 0, st, a, plan, n_tiles, run);
  else hipLaunchKernelGGL((swiglu_kernel<BITS, 128, SBQ>), grid, dim3(kGemmThreads), 0, st, a, plan, n_tiles, run);
  return hipGetLastError();
}

// Quad scale loads (8 bytes per column, four groups of 64): the expert and
// column offsets of the scales are multiples of 8 bytes when k / 64 is a
// multiple of 4, so only the arrays' own alignment is checked.
static bool sbq_ok(int k, int group_size, const void* s, const void* b) {
  return (k / 64) % 4 == 0 && group_size == 64 && ((uintptr_t)s & 7) == 0 && ((uintptr_t)b & 7) == 0;
}

template <int BITS>
static hipError_t launch_swiglu_bits(const SwigluArgs& a, const int32_t* plan, hipStream_t st) {
  if constexpr (BITS == 16) {
    return launch_swiglu_sbq<16, false>(a, plan, st);
  } else {
    return sbq_ok(a.k, a.group_size, a.sg, a.bg) && sbq_ok(a.k, a.group_size, a.su, a.bu)
               ? launch_swiglu_sbq<BITS, true>(a, plan, st)
               : launch_swiglu_sbq<BITS, false>(a, plan, st);
  }
}

// Row tile from the mean number of pairs per expert.  Measured on the
// Qwen3-30B-A3B-shaped layers (128 experts, top-8) with the XCD-aware
// workgroup order above: at 2048 tokens (128 pairs per expert on average,
// 100 to 159) 64-row tiles beat 160-row ones for gate (92.7 vs 94.3 us),
// down (103.5 vs 113.2) and the fused gate/up (193.1 vs 197.8): two or
// three row tiles per expert give the chip more workgroups than one
// 160-row tile, and the repeated weight columns mostly come from L2 or the
// last-level cache.  At 512 tokens (32 per expert) 64 rows are best too;
// 32 rows below 16 per expert, 128 above 160 per expert (each expert's
// weights then stream once per 128 pairs).  Column tile of the plain
// grouped GEMM: 256 columns (nb = 2) over interleaved scales from 64 pairs
// per expert on average, where it measured 5-7 % faster than 128 (2048
// tokens: gate 100.8 vs 107.2 us, up 100.6 vs 108.2, down 115.8 vs 122.1;
// 1024 tokens: gate 69.1 vs 74.8, down 77.0 vs 79.6); at 512 tokens (32 per
// expert) and over row-major scales 128 columns stay faster, as the wider
// tile halves the workgroups per expert.
// QMM_MOE_FORCE="bm,nb" overrides the tile (tuning sweeps).  The bucketing
// and the grouped GEMM must agree on it, so both take it from here.
// QMM_MOE_FORCE is read on every call (tuning sweeps change it between
// calls); a routing plan built under one value and used under another is
// caught on the device by the plan-header check (the output becomes NaN).
static void moe_tile(int pairs, int experts, int stiled, int* bm_out, int* nb_out) {
  const int mean = (pairs + experts - 1) / experts;
  int bm = mean <= 16 ? 32 : mean <= 160 ? 64 : 128;
  int nb = stiled && bm == 64 && mean >= 64 ? 2 : 1;
  if (const char* env = getenv("QMM_MOE_FORCE")) {
    int fb = 0, fn = 0;
    if (sscanf(env, "%d,%d", &fb, &fn) == 2 && (fb == 32 || fb == 64 || fb == 128 || (fb == 160 && fn == 1)) &&
        (fn == 1 || fn == 2)) {
      bm = fb;
      nb = fn;
    }
  }
  *bm_out = bm;
  *nb_out = nb;
}

// ---------------------------------------------------------------------------
// Static device scratch of the allocation-free grouped GEMM
// (qmm_qgemm_grouped_noalloc): the bucket lists and tile list that
// qmm_qgemm_grouped keeps in its caller's workspace live here instead.  Each
// GPU the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is passed to kernels.  Every call on one GPU shares the
// array, so calls that overlap on one GPU race; nothing in it needs to start
// at zero (the bucketing writes every word the GEMM reads).
static __device__ __align__(256) unsigned char scratch[kGroupedScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t grouped_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_moe_route(const int32_t* ids, int t, int top_k, int e, void* plan, hipStream_t st) {
  int bm, nb;  // the routing plan depends on the row tile only
  moe_tile(t * top_k, e, 0, &bm, &nb);
  return launch_bucket(ids, t * top_k, e, bm, reinterpret_cast<int32_t*>(plan), st);
}

template <int BITS, int BM, int NB, bool SBQ>
static hipError_t launch_grouped_tile(const GroupedArgs& a, int32_t* ws, bool bucket, hipStream_t st) {
  constexpr int BN = 4 * NB * 32;
  const int pairs = a.t * a.top_k;
  if (bucket) {
    hipError_t err = launch_bucket(a.ids, pairs, a.e, BM, ws, st);
    if (err != hipSuccess) return err;
  }
  const int n_tiles = (a.n + BN - 1) / BN;
  const int m_tiles = max_row_tiles(pairs, a.e, BM);
  const int run = kMoeRun;
  hipLaunchKernelGGL((grouped_kernel<BITS, BM, NB, SBQ>), dim3(moe_grid(m_tiles, n_tiles, run)), dim3(kGemmThreads),
                     0, st, a, ws, n_tiles, run);
  return hipGetLastError();
}

template <int BITS, bool SBQ>
static hipError_t launch_grouped_sbq(const GroupedArgs& a, int32_t* ws, bool bucket, hipStream_t st) {
  int bm, nb;
  moe_tile(a.t * a.top_k, a.e, a.stiled, &bm, &nb);
  if constexpr (BITS == 16) {  // fp16 weights: one column block per wave, no scales
    if (bm == 32) return launch_grouped_tile<16, 32, 1, false>(a, ws, bucket, st);
    if (bm == 64) return launch_grouped_tile<16, 64, 1, false>(a, ws, bucket, st);
    if (bm == 160) return launch_grouped_tile<16, 160, 1, false>(a, ws, bucket, st);
    return launch_grouped_tile<16, 128, 1, false>(a, ws, bucket, st);
  } else {
    if (bm == 32) return nb == 2 ? launch_grouped_tile<BITS, 32, 2, SBQ>(a, ws, bucket, st) : launch_grouped_tile<BITS, 32, 1, SBQ>(a, ws, bucket, st);
    if (bm == 64) return nb == 2 ? launch_grouped_tile<BITS, 64, 2, SBQ>(a, ws, bucket, st) : launch_grouped_tile<BITS, 64, 1, SBQ>(a, ws, bucket, st);
    if (bm == 160) return launch_grouped_tile<BITS, 160, 1, SBQ>(a, ws, bucket, st);
    return nb == 2 ? launch_grouped_tile<BITS, 128, 2, SBQ>(a, ws, bucket, st) : launch_grouped_tile<BITS, 128, 1, SBQ>(a, ws, bucket, st);
  }
}

template <int BITS>
static hipError_t launch_grouped_bits(const GroupedArgs& a, int32_t* ws, bool bucket, hipStream_t st) {
  if constexpr (BITS == 16) return launch_grouped_sbq<16, false>(a, ws, bucket, st);
  return sbq_ok(a.k, a.group_size, a.s, a.b) ? launch_grouped_sbq<BITS, true>(a, ws, bucket, st)
                                             : launch_grouped_sbq<BITS, false>(a, ws, bucket, st);
}

hipError_t launch_qgemm_grouped(const GroupedArgs& a, int bits, void* ws, bool bucket, hipStream_t st) {
  int32_t* w = reinterpret_cast<int32_t*>(ws);
  switch (bits) {
    case 2: return launch_grouped_bits<2>(a, w, bucket, st);
    case 3: return launch_grouped_bits<3>(a, w, bucket, st);
    case 4: return launch_grouped_bits<4>(a, w, bucket, st);
    case 5: return launch_grouped_bits<5>(a, w, bucket, st);
    case 6: return launch_grouped_bits<6>(a, w, bucket, st);
    case 8: return launch_grouped_bits<8>(a, w, bucket, st);
    case 16: return launch_grouped_bits<16>(a, w, bucket, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_moe_swiglu(const uint32_t* wg, const uint16_t* sg, const uint16_t* bg,
                             const uint32_t* wu, const uint16_t* su, const uint16_t* bu,
                             const uint16_t* x, const void* plan, uint16_t* h, int t, int top_k,
                             int e, int n, int k, int bits, int group_size, int wtiled, int stiled,
                             hipStream_t st) {
  const SwigluArgs a{wg, sg, bg, wu, su, bu, x, h, t, top_k, e, n, k, group_size, wtiled, stiled};
  const int32_t* p = static_cast<const int32_t*>(plan);
  switch (bits) {
    case 2: return launch_swiglu_bits<2>(a, p, st);
    case 3: return launch_swiglu_bits<3>(a, p, st);
    case 4: return launch_swiglu_bits<4>(a, p, st);
    case 5: return launch_swiglu_bits<5>(a, p, st);
    case 6: return launch_swiglu_bits<6>(a, p, st);
    case 8: return launch_swiglu_bits<8>(a, p, st);
    case 16: return launch_swiglu_bits<16>(a, p, st);
    default: return hipErrorInvalidValue;
  }
}

// y[t, :] = sum over j of weights[t, j] * y_pairs[t * top_k + j, :], the
// slots added in order j = 0 .. top_k-1 (fp32 fma): the routing-weighted
// combine of the down projection's per-pair rows, independent of scheduling.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ y_pairs,
                                                          const float* __restrict__ weights,
                                                          float* __restrict__ y, int t, int top_k,
                                                          int n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)t * n) return;
  const long tok = i / n;
  const long col = i % n;
  float acc = 0.0f;
  for (int j = 0; j < top_k; ++j)
    acc = fmaf(weights[tok * top_k + j], y_pairs[(tok * top_k + j) * n + col], acc);
  y[i] = acc;
}

// The same over four adjacent columns per thread (16-byte loads and stores;
// n a multiple of 4, both row arrays 16-byte aligned): each column's sum is
// formed exactly as above, so the results are bit-identical.
__global__ __launch_bounds__(256) void moe_combine4_kernel(const float4* __restrict__ y_pairs,
                                                           const float* __restrict__ weights,
                                                           float4* __restrict__ y, int t, int top_k,
                                                           int n4) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)t * n4) return;
  const long tok = i / n4;
  const long col = i % n4;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 8
  for (int j = 0; j < top_k; ++j) {
    const float w = weights[tok * top_k + j];
    const float4 v = y_pairs[(tok * top_k + j) * n4 + col];
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  y[i] = acc;
}

hipError_t launch_moe_combine(const float* y_pairs, const float* weights, float* y, int t, int top_k,
                              int n, hipStream_t st) {
  if (n % 4 == 0 && reinterpret_cast<uintptr_t>(y_pairs) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0) {
    const long count = (long)t * (n / 4);
    hipLaunchKernelGGL(moe_combine4_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<const float4*>(y_pairs), weights, reinterpret_cast<float4*>(y), t,
                       top_k, n / 4);
    return hipGetLastError();
  }
  const long count = (long)t * n;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                     y_pairs, weights, y, t, top_k, n);
  return hipGetLastError();
}

}  // namespace qmm
