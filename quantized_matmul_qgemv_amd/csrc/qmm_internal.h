// Host-side interfaces between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmm {

struct GemvProblem {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  const uint16_t* x;
  float* y;
  int32_t n;
  int32_t k;
};

// One workgroup's share of a batched GEMV: rows [row0, row0 + nrows) of a
// problem.  64 bytes, read once per workgroup.
struct alignas(64) GemvBlock {
  GemvProblem p;
  int32_t row0;
  int32_t nrows;
  int32_t pad[2];
};
static_assert(sizeof(GemvBlock) == 64, "GemvBlock must stay 64 bytes");

// Host image header of a batched-GEMV plan (64 bytes, followed by the
// GemvBlock records).
struct alignas(64) GemvPlanHeader {
  uint32_t magic;       // 'QMMP'
  uint32_t version;
  int32_t bits;
  int32_t group_size;
  int32_t lanes_per_row;
  int32_t rows_per_block;  // rows per workgroup pass
  int32_t num_blocks;
  int32_t max_groups;
  int32_t count;
  int32_t pad[7];
};
static_assert(sizeof(GemvPlanHeader) == 64, "plan header must stay 64 bytes");
constexpr uint32_t kPlanMagic = 0x504D4D51u;  // "QMMP"
constexpr uint32_t kPlanVersion = 1;

// Launch geometry chosen for a GEMV.
struct GemvGeom {
  int lanes_per_row;  // lanes cooperating on one row (power of two <= 16)
  int row_unroll;     // rows per lane slot held in flight
  int wave_ksplit;    // waves of a workgroup splitting one row's groups
  int rows_per_pass;  // rows one pass of a workgroup covers
  int passes;         // passes per workgroup (rows per workgroup = passes * rows_per_pass)
};

GemvGeom gemv_choose(int n, int k, int bits);
int gemv_row_unroll(int bits);
int gemv_rows_per_pass(int lanes_per_row, int row_unroll, int wave_ksplit);
int gemv_lanes_for_groups(int groups);
size_t gemv_lds_bytes(int max_groups, const GemvGeom& g);

hipError_t launch_qgemv(const GemvProblem& p, int bits, int group_size, const GemvGeom& g,
                        hipStream_t st);
hipError_t launch_qgemv_batched(const GemvBlock* blocks, int num_blocks, int bits, int group_size,
                                int lanes_per_row, int max_groups, hipStream_t st);

struct GemmArgs {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  const uint16_t* x;
  float* y;
  int m, n, k;
  int group_size;  // codes per scale/bias group: 32, 64 or 128
  int wtiled;      // weights in the tile-interleaved layout (qmm_repack_tiled)
  int stiled;      // scales and biases interleaved (qmm_repack_scales_tiled; s holds both)
};
size_t gemm_workspace_bytes(int m, int n, int k, int bits);
hipError_t launch_qgemm(const GemmArgs& a, int bits, void* workspace, hipStream_t st);

// Batched GEMM plan image: header, problem table, tile records.
struct alignas(64) GemmBatchProblem {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  const uint16_t* x;
  float* y;
  int32_t m, n, k;
  int32_t pad[3];
};
static_assert(sizeof(GemmBatchProblem) == 64, "GemmBatchProblem must stay 64 bytes");

// One workgroup: output tile (m0, n0) of a problem, groups [g0, g1).  With
// splits > 1 the tile's fp32 partial goes to workspace slot
// sid * splits + split (bm x bn floats, row-major); a reduce kernel sums the
// slots of each split tile in split order into y.  problem < 0: no work.
struct GemmTileRec {
  int32_t problem;
  int32_t m0, n0;
  int32_t g0, g1;
  int32_t split, splits;
  int32_t sid;
};
static_assert(sizeof(GemmTileRec) == 32, "GemmTileRec must stay 32 bytes");

// Split tile sid: where its sum goes.
struct GemmSplitTile {
  int32_t problem, m0, n0, pad;
};

struct alignas(64) GemmBatchHeader {
  uint32_t magic;        // 'QMMB'
  uint32_t version;
  int32_t bits;
  int32_t group_size;
  int32_t bm, nb;        // tile: bm rows x (nb * 128) columns
  int32_t sbq;           // every k range is a multiple of 4 groups
  int32_t count;         // problems
  int32_t num_tiles;     // tile records (grid size)
  int32_t split_tiles;   // tiles whose k is split (GemmSplitTile records after the tiles)
  int32_t splits;
  int32_t wtiled;        // weights in the tile-interleaved layout (qmm_repack_tiled)
  uint64_t workspace_bytes;
  int32_t kw;            // k halves per workgroup (1, or 2 with 8 waves)
  int32_t stiled;        // scales and biases interleaved (qmm_repack_scales_tiled)
};
static_assert(sizeof(GemmBatchHeader) == 64, "GemmBatchHeader must stay 64 bytes");
constexpr uint32_t kBatchMagic = 0x424D4D51u;  // "QMMB"
constexpr uint32_t kBatchVersion = 1;

// Tile and split count for one GEMM (k split evenly), from the batch planner's
// cost model; honours QMM_GEMM_FORCE.
void gemm_choose(int m, int n, int k, int bits, int* bm, int* nb, int* splits);

// Choose the tile and split count for a batch and write the plan image.
// Returns the image size; writes nothing when out is null or too small.
size_t gemm_batch_build(const GemmBatchProblem* probs, int count, int bits, int group_size,
                        int wtiled, int stiled, void* out, size_t out_bytes);
hipError_t launch_qgemm_batched(const void* plan_device, const GemmBatchHeader& hdr,
                                void* workspace, hipStream_t st);

struct GroupedArgs {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  const uint16_t* a;
  int a_row_per_pair;
  const int32_t* ids;
  float* y;
  int t, top_k, e, n, k;
  int group_size;
  int wtiled;  // weights in the tile-interleaved layout (qmm_repack_tiled)
  int stiled;  // scales and biases interleaved (qmm_repack_scales_tiled; s holds both)
};
size_t grouped_workspace_bytes(int t, int top_k, int e, int n);
// Static device scratch of the allocation-free grouped GEMM: its size, and
// its device address on the current device (looked up once per device).
constexpr size_t kGroupedScratchBytes = 1u << 20;
hipError_t grouped_scratch(void** ptr);
// bucket = false: ws already holds a routing plan for these ids (launch_moe_route).
hipError_t launch_qgemm_grouped(const GroupedArgs& a, int bits, void* ws, bool bucket, hipStream_t st);
hipError_t launch_moe_route(const int32_t* ids, int t, int top_k, int e, void* plan, hipStream_t st);
hipError_t launch_moe_swiglu(const uint32_t* wg, const uint16_t* sg, const uint16_t* bg,
                             const uint32_t* wu, const uint16_t* su, const uint16_t* bu,
                             const uint16_t* x, const void* plan, uint16_t* h, int t, int top_k,
                             int e, int n, int k, int bits, int group_size, int wtiled, int stiled,
                             hipStream_t st);
hipError_t launch_moe_combine(const float* y_pairs, const float* weights, float* y, int t, int top_k,
                              int n, hipStream_t st);

hipError_t launch_quantize(const float* w, uint32_t* words, uint16_t* s, uint16_t* b, int n,
                           int k, int bits, int group_size, hipStream_t st);
hipError_t launch_convert_bf16(const uint16_t* src, uint16_t* dst, long count, hipStream_t st);
hipError_t launch_repack_tiled(const uint32_t* w, uint32_t* out, int n, int k, int bits, hipStream_t st);
hipError_t launch_repack_scales_tiled(const uint16_t* s, const uint16_t* b, uint16_t* out, int n, int k,
                                      hipStream_t st);
hipError_t launch_unpack_codes(const uint32_t* w, uint8_t* codes, int n, int k, int bits,
                               hipStream_t st);
hipError_t launch_dequant(const uint32_t* w, const uint16_t* s, const uint16_t* b, void* out,
                          int out_is_f16, int n, int k, int bits, int group_size, hipStream_t st);

}  // namespace qmm
