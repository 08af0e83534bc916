// Batched prefill GEMM: several independent y_p = x_p W_hat_p^T in one
// launch (BaseRT, native-Metal LLM inference on Apple Silicon, §3.4: prefill
// as tiled GEMMs; §3.3: dequantization inside the inner loop).  The
// projections of a transformer layer that read the same activations (q, k
// and v; gate and up) are independent, and one grid over all their tiles
// fills the 256 CUs where each alone would leave part of the chip idle.
//
// A host-built plan lists one record per workgroup: problem, output tile,
// k range.  When the planner splits k, every split writes its fp32 partial
// tile to the workspace and a second, short kernel adds the partials of
// each tile in split order into y, so results do not depend on scheduling.
// (Summing inside the GEMM kernel, by the last split to finish, needs
// device-scope coherence between the 8 XCDs' L2 caches: either cache-wide
// write-back/invalidate or uncached partial traffic, both measured slower
// than the extra launch.)
//
// Workgroups are dealt round-robin to the 8 XCDs; records are laid out so
// that each XCD gets a contiguous run of the logical order (row tiles of
// one column tile next to each other), which keeps a column tile's weights
// in one L2.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qgemm_core.h"
#include "qgemm_wide.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int kXcdCount = 8;

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// y tile of split tile `sid` = sum of its partial tiles in split order.
// One workgroup reduces 1024 outputs of one tile (4 per thread, 16-byte
// loads of every partial issued together).
// The split count is a template argument so that all S partial loads of a
// thread are issued before the first addition (with a run-time trip count
// each load waited for the previous sum: S memory latencies in a row); the
// sum is still taken in split order 0, 1, ..., S-1.  S = 0: the count is
// the run-time `splits` (a forced split count the planner never chooses).
template <int S>
__global__ __launch_bounds__(256) void qgemm_batched_reduce_kernel(
    const GemmBatchProblem* __restrict__ probs, const GemmSplitTile* __restrict__ st,
    const float* __restrict__ partials, int bm, int bn, int splits) {
  const int per_tile = bm * bn / 1024;
  const int sid = blockIdx.x / per_tile;
  const int e0 = (blockIdx.x % per_tile) * 1024 + threadIdx.x * 4;
  const GemmSplitTile t = st[sid];
  const GemmBatchProblem P = probs[t.problem];
  const int ns = S > 0 ? S : splits;
  const gptr<float4_t> src = reinterpret_cast<gptr<float4_t>>(to_global(partials)) +
                             ((size_t)sid * ns * bm * bn + e0) / 4;
  const size_t stride = (size_t)bm * bn / 4;
  float4_t acc;
  if constexpr (S > 0) {
    float4_t v[S];
#pragma unroll
    for (int sp = 0; sp < S; ++sp) v[sp] = src[sp * stride];
    acc = v[0];
#pragma unroll
    for (int sp = 1; sp < S; ++sp) acc += v[sp];
  } else {
    acc = src[0];
    for (int sp = 1; sp < splits; ++sp) acc += src[sp * stride];
  }
  const int r = e0 / bn;
  const int c = e0 % bn;
  const int row = t.m0 + r;
  if (row >= P.m) return;
  const gptr_mut<float> y = to_global_mut(P.y) + (size_t)row * P.n + t.n0 + c;
  const int cols = P.n - t.n0 - c;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < cols) y[q] = acc[q];
}

template <int BITS, int BM, int NB, bool SBQ, int KW>
__global__ __launch_bounds__(kGemmThreads * KW) __attribute__((amdgpu_waves_per_eu(2))) void qgemm_batched_kernel(
    const GemmBatchProblem* __restrict__ probs, const GemmTileRec* __restrict__ tiles,
    float* partials, int gs, int wtiled, int stiled) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[gemm_lds_halves(BM, NB, KW)];
  constexpr int BN = 4 * NB * 32;
  const GemmTileRec t = tiles[blockIdx.x];
  if (t.problem < 0) return;
  const GemmBatchProblem P = probs[t.problem];
  const int m = P.m;
  const int m0 = t.m0;
  const bool split = t.splits > 1;
  float* ytile = split ? partials + ((size_t)t.sid * t.splits + t.split) * (BM * BN) : P.y + t.n0;
  const int ldy = split ? BN : P.n;
  const int rowoff = split ? 0 : m0;
  auto a_row = [&](int i) { const int r = m0 + i; return r < m ? r : m - 1; };
  auto c_row = [&](int i) { return m0 + i < m ? rowoff + i : -1; };
  gemm_tile<BITS, BM, NB, SBQ, false, KW>(ARows{P.x, P.k}, a_row, c_row, P.w, P.s, P.b, ytile, ldy, t.n0,
                               P.n, t.g0, t.g1, lds, gs, nullptr, nullptr, nullptr, nullptr, wtiled, stiled);
}

template <int BITS, bool SBQ>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(1))) void qgemm_batched_wide_kernel(
    const GemmBatchProblem* __restrict__ probs, const GemmTileRec* __restrict__ tiles,
    float* partials, int gs, int wtiled, int stiled) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kWideLdsHalves];
  constexpr int BM = kWideBM;
  constexpr int BN = 256;
  const GemmTileRec t = tiles[blockIdx.x];
  if (t.problem < 0) return;
  const GemmBatchProblem P = probs[t.problem];
  const int m = P.m;
  const int m0 = t.m0;
  const bool split = t.splits > 1;
  float* ytile = split ? partials + ((size_t)t.sid * t.splits + t.split) * (BM * BN) : P.y + t.n0;
  const int ldy = split ? BN : P.n;
  const int rowoff = split ? 0 : m0;
  auto a_row = [&](int i) { const int r = m0 + i; return r < m ? r : m - 1; };
  auto c_row = [&](int i) { return m0 + i < m ? rowoff + i : -1; };
  gemm_tile_wide<BITS, SBQ>(ARows{P.x, P.k}, a_row, c_row, P.w, P.s, P.b, ytile, ldy, t.n0, P.n,
                            t.g0, t.g1, lds, gs, wtiled, stiled);
}

// ------------------------------------------------------------------ host --

// Tile configurations and the planner's cost model.  For a batch with W
// workgroups (tiles x splits), each running `steps` k64 steps (per k half),
// on a configuration with `occ` resident workgroups per CU:
//   k       = ceil(W / 256)                  workgroups on the busiest CU
//   compute = steps * t1 * ceil(k / occ) * min(k, occ)^gamma
//   l2      = W * steps * kw * (bm * 128 + bn * 8 * bits) / kL2GBs
//   time    = kFixedUs + max(compute, l2) + (splits > 1 ? split cost : 0)
// t1 is the time of one step of a workgroup alone on a CU; gamma says how
// much a CU's resident workgroups slow each other down (0: not at all, 1:
// they take turns); the l2 term bounds the operand traffic of the whole
// grid (A tiles and packed weights per step, from L2).  t1, gamma,
// kFixedUs and kL2GBs were fitted (least squares on log time) to about
// 1,100 launches of the Qwen3-4B-shaped prefill groups (q+k+v, o, gate+up,
// down) at M = 128 ... 2048 with 4-bit weights, every configuration and
// split count, each launch reading its weights from HBM (rotating over 8
// layers): the fit's rms error is 7-12 % per configuration, and its choice
// is within 3 % of the best measured configuration at every M.
struct TileCfg {
  int bm, nb, kw, occ;
  double t1_us, gamma;
};
constexpr TileCfg kCfgs[] = {
    {256, 2, 1, 1, 1.900, 0.00}, {128, 2, 1, 2, 1.040, 0.48}, {128, 1, 1, 3, 0.680, 0.48},
    {64, 2, 1, 3, 0.600, 0.64},  {64, 1, 1, 4, 0.400, 0.48},  {32, 2, 1, 3, 0.460, 0.64},
    {32, 1, 1, 5, 0.320, 0.52},
    // two k halves per workgroup (8 waves)
    {128, 1, 2, 1, 1.320, 0.00}, {64, 2, 2, 1, 1.240, 0.00}, {64, 1, 2, 2, 0.720, 0.64},
    {32, 1, 2, 2, 0.580, 0.64},
};
constexpr int kCUs = 256;
constexpr double kFixedUs = 1.0;
constexpr double kL2GBs = 10000.0;
constexpr int kSplitChoices[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16};
constexpr double kSplitUs = 6.25;          // reduce launch
constexpr double kSplitUsPerMB = 0.5;      // partial tiles written and read back
constexpr double kMaxPartialBytes = 512.0 * 1024 * 1024;

int ceil_div_i(long a, long b) { return (int)((a + b - 1) / b); }

struct Choice {
  int cfg, splits;
  bool sbq;
  double us;
};

// Group boundary of split s out of S over G groups; multiples of 4 when sbq.
int split_bound(int s, int S, int G, bool sbq) {
  if (s >= S) return G;
  const long g = (long)s * G / S;
  return sbq ? (int)(g / 4 * 4) : (int)g;
}

bool sbq_ok(const GemmBatchProblem* probs, int count, int S) {
  for (int p = 0; p < count; ++p) {
    const int G = probs[p].k / 64;
    if (G % 4 != 0 || G / S < 4) return false;
  }
  return true;
}

bool splits_ok(const GemmBatchProblem* probs, int count, int S) {
  for (int p = 0; p < count; ++p)
    if (probs[p].k / 64 < S) return false;
  return true;
}

// divisible: only split counts that divide every problem's group count
// and one k half per workgroup (the single-GEMM kernel).
// f16w: unquantized fp16 weights hold 4x the register bytes of a 4-bit
// weight ring, so only the one-column-block tiles (nb = 1) are used.  The
// same holds for 5- to 8-bit weights (1.25-2x): on the 2048 x 9728 x 2560
// GEMM their two-column-block tiles measured 5-20 % slower than 128 x 128
// (the cost model's constants come from 4-bit launches).
Choice choose(const GemmBatchProblem* probs, int count, int bits, bool divisible, bool f16w) {
  Choice best{2, 1, false, 1e300};
  for (int ci = 0; ci < (int)(sizeof kCfgs / sizeof kCfgs[0]); ++ci) {
    const TileCfg& c = kCfgs[ci];
    if ((f16w || bits >= 5) && c.nb != 1) continue;
    if (divisible && c.kw != 1) continue;
    const int bn = c.nb * 128;
    for (int S : kSplitChoices) {
      if (!splits_ok(probs, count, S * c.kw)) continue;
      bool even = true;
      for (int p = 0; p < count; ++p) even = even && (probs[p].k / 64) % S == 0;
      if (divisible && !even) continue;
      long wg = 0;
      int steps = 0;
      for (int p = 0; p < count; ++p) {
        const long tp = (long)ceil_div_i(probs[p].m, c.bm) * ceil_div_i(probs[p].n, bn);
        wg += tp * S;
        const int st = ceil_div_i(ceil_div_i(probs[p].k / 64, S), c.kw);
        if (st > steps) steps = st;
      }
      if (wg == 0) continue;
      const double partial = S > 1 ? (double)wg * c.bm * bn * 4.0 : 0.0;
      if (partial > kMaxPartialBytes) continue;
      const long k = (wg + kCUs - 1) / kCUs;
      const double compute = steps * c.t1_us * (double)((k + c.occ - 1) / c.occ) *
                             pow((double)(k < c.occ ? k : c.occ), c.gamma);
      const double l2 = (double)wg * steps * c.kw * (c.bm * 128.0 + bn * 8.0 * bits) / (kL2GBs * 1e3);
      const double us = kFixedUs + (compute > l2 ? compute : l2) +
                        (S > 1 ? kSplitUs + kSplitUsPerMB * partial / 1e6 : 0.0);
      if (us < best.us * 0.999) best = Choice{ci, S, sbq_ok(probs, count, S), us};
    }
  }
  // QMM_GEMM_FORCE="bm,nb,splits[,kw]" overrides the choice (tuning
  // sweeps); it is ignored unless it names a configuration and a valid
  // split count.
  if (const char* env = getenv("QMM_GEMM_FORCE")) {
    int bm = 0, nb = 0, sp = 0, kw = 1;
    const int got = sscanf(env, "%d,%d,%d,%d", &bm, &nb, &sp, &kw);
    const bool parsed = got >= 3 && sp >= 1 && (kw == 1 || kw == 2);
    bool even = parsed;
    for (int p = 0; parsed && p < count; ++p) even = even && (probs[p].k / 64) % sp == 0;
    if (parsed && splits_ok(probs, count, sp * kw) && (even || !divisible)) {
      for (int ci = 0; ci < (int)(sizeof kCfgs / sizeof kCfgs[0]); ++ci)
        if (kCfgs[ci].bm == bm && kCfgs[ci].nb == nb && kCfgs[ci].kw == kw && (!f16w || nb == 1))
          best = Choice{ci, sp, sbq_ok(probs, count, sp), 0.0};
    }
  }
  return best;
}

}  // namespace

void gemm_choose(int m, int n, int k, int bits, int* bm, int* nb, int* splits) {
  GemmBatchProblem p;
  memset(&p, 0, sizeof p);
  p.m = m;
  p.n = n;
  p.k = k;
  const Choice ch = choose(&p, 1, bits, true, bits == 16);
  *bm = kCfgs[ch.cfg].bm;
  *nb = kCfgs[ch.cfg].nb;
  *splits = ch.splits;
}

size_t gemm_batch_build(const GemmBatchProblem* probs, int count, int bits, int group_size,
                        int wtiled, int stiled, void* out, size_t out_bytes) {
  Choice ch = choose(probs, count, bits, false, bits == 16);
  // quad scale loads (8 bytes per column): groups of 64 with 8-byte aligned
  // scale and bias arrays only
  bool sb_aligned = true;
  for (int p = 0; p < count; ++p)
    sb_aligned = sb_aligned && ((uintptr_t)probs[p].s & 7) == 0 && ((uintptr_t)probs[p].b & 7) == 0;
  ch.sbq = ch.sbq && group_size == 64 && bits != 16 && sb_aligned;
  const TileCfg& c = kCfgs[ch.cfg];
  const int bn = c.nb * 128;
  const int S = ch.splits;
  long logical = 0, split_tiles = 0;
  for (int p = 0; p < count; ++p) {
    const long tp = (long)ceil_div_i(probs[p].m, c.bm) * ceil_div_i(probs[p].n, bn);
    logical += tp * S;
    if (S > 1) split_tiles += tp;
  }
  const long per = (logical + kXcdCount - 1) / kXcdCount;
  const long grid = per * kXcdCount;
  const size_t need = sizeof(GemmBatchHeader) + (size_t)count * sizeof(GemmBatchProblem) +
                      (size_t)grid * sizeof(GemmTileRec) + (size_t)split_tiles * sizeof(GemmSplitTile);
  if (out == nullptr || out_bytes < need) return need;

  GemmBatchHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.magic = kBatchMagic;
  hdr.version = kBatchVersion;
  hdr.bits = bits;
  hdr.group_size = group_size;
  hdr.bm = c.bm;
  hdr.nb = c.nb;
  hdr.kw = c.kw;
  hdr.sbq = ch.sbq ? 1 : 0;
  hdr.count = count;
  hdr.num_tiles = (int32_t)grid;
  hdr.split_tiles = (int32_t)split_tiles;
  hdr.splits = S;
  hdr.wtiled = wtiled ? 1 : 0;
  hdr.stiled = stiled ? 1 : 0;
  hdr.workspace_bytes = S > 1 ? (size_t)split_tiles * S * c.bm * bn * 4 : 0;
  unsigned char* base = static_cast<unsigned char*>(out);
  memcpy(base, &hdr, sizeof hdr);
  memcpy(base + sizeof hdr, probs, (size_t)count * sizeof(GemmBatchProblem));
  GemmTileRec* recs = reinterpret_cast<GemmTileRec*>(base + sizeof hdr + (size_t)count * sizeof(GemmBatchProblem));
  GemmSplitTile* sts = reinterpret_cast<GemmSplitTile*>(recs + grid);
  for (long i = 0; i < grid; ++i) recs[i] = GemmTileRec{-1, 0, 0, 0, 0, 0, 1, 0};
  // logical order: problem, column tile, split, row tile (row tiles of one
  // column tile adjacent); logical index L goes to XCD L / per, position
  // L % per inside it, i.e. workgroup (L % per) * 8 + L / per.
  long L = 0;
  int sid = 0;
  for (int p = 0; p < count; ++p) {
    const GemmBatchProblem& q = probs[p];
    const int G = q.k / 64;
    const int mt = ceil_div_i(q.m, c.bm), nt = ceil_div_i(q.n, bn);
    for (int tn = 0; tn < nt; ++tn) {
      for (int s = 0; s < S; ++s) {
        for (int tm = 0; tm < mt; ++tm) {
          GemmTileRec r;
          r.problem = p;
          r.m0 = tm * c.bm;
          r.n0 = tn * bn;
          r.g0 = split_bound(s, S, G, ch.sbq);
          r.g1 = split_bound(s + 1, S, G, ch.sbq);
          r.split = s;
          r.splits = S;
          r.sid = S > 1 ? sid + tm : 0;
          recs[(L % per) * kXcdCount + L / per] = r;
          ++L;
        }
      }
      if (S > 1) {
        for (int tm = 0; tm < mt; ++tm) sts[sid + tm] = GemmSplitTile{p, tm * c.bm, tn * bn, 0};
        sid += mt;
      }
    }
  }
  return need;
}

template <int BITS, int BM, int NB, int KW = 1>
static void launch_batched_cfg(const GemmBatchProblem* probs, const GemmTileRec* tiles,
                               const GemmBatchHeader& h, float* partials, hipStream_t st) {
  if (h.sbq)
    hipLaunchKernelGGL((qgemm_batched_kernel<BITS, BM, NB, true, KW>), dim3(h.num_tiles),
                       dim3(kGemmThreads * KW), 0, st, probs, tiles, partials, h.group_size, h.wtiled, h.stiled);
  else
    hipLaunchKernelGGL((qgemm_batched_kernel<BITS, BM, NB, false, KW>), dim3(h.num_tiles),
                       dim3(kGemmThreads * KW), 0, st, probs, tiles, partials, h.group_size, h.wtiled, h.stiled);
}

template <int BITS>
static void launch_batched_bits(const GemmBatchProblem* probs, const GemmTileRec* tiles,
                                const GemmBatchHeader& h, float* partials, hipStream_t st) {
  if constexpr (BITS == 16) {  // nb = 1 tiles only (see choose)
    if (h.kw == 2) {
      if (h.bm == 128) launch_batched_cfg<16, 128, 1, 2>(probs, tiles, h, partials, st);
      else if (h.bm == 64) launch_batched_cfg<16, 64, 1, 2>(probs, tiles, h, partials, st);
      else launch_batched_cfg<16, 32, 1, 2>(probs, tiles, h, partials, st);
    } else if (h.bm == 128) launch_batched_cfg<16, 128, 1>(probs, tiles, h, partials, st);
    else if (h.bm == 64) launch_batched_cfg<16, 64, 1>(probs, tiles, h, partials, st);
    else launch_batched_cfg<16, 32, 1>(probs, tiles, h, partials, st);
    return;
  } else {
    if (h.kw == 2) {
      if (h.bm == 128) launch_batched_cfg<BITS, 128, 1, 2>(probs, tiles, h, partials, st);
      else if (h.bm == 64 && h.nb == 2) launch_batched_cfg<BITS, 64, 2, 2>(probs, tiles, h, partials, st);
      else if (h.bm == 64) launch_batched_cfg<BITS, 64, 1, 2>(probs, tiles, h, partials, st);
      else launch_batched_cfg<BITS, 32, 1, 2>(probs, tiles, h, partials, st);
    } else if (h.bm == 256) {
      if (h.sbq)
        hipLaunchKernelGGL((qgemm_batched_wide_kernel<BITS, true>), dim3(h.num_tiles), dim3(kGemmThreads),
                           0, st, probs, tiles, partials, h.group_size, h.wtiled, h.stiled);
      else
        hipLaunchKernelGGL((qgemm_batched_wide_kernel<BITS, false>), dim3(h.num_tiles), dim3(kGemmThreads),
                           0, st, probs, tiles, partials, h.group_size, h.wtiled, h.stiled);
    } else if (h.bm == 128) {
      if (h.nb == 2) launch_batched_cfg<BITS, 128, 2>(probs, tiles, h, partials, st);
      else launch_batched_cfg<BITS, 128, 1>(probs, tiles, h, partials, st);
    } else if (h.bm == 64) {
      if (h.nb == 2) launch_batched_cfg<BITS, 64, 2>(probs, tiles, h, partials, st);
      else launch_batched_cfg<BITS, 64, 1>(probs, tiles, h, partials, st);
    } else {
      if (h.nb == 2) launch_batched_cfg<BITS, 32, 2>(probs, tiles, h, partials, st);
      else launch_batched_cfg<BITS, 32, 1>(probs, tiles, h, partials, st);
    }
  }
}

hipError_t launch_qgemm_batched(const void* plan_device, const GemmBatchHeader& h, void* workspace,
                                hipStream_t st) {
  const unsigned char* base = static_cast<const unsigned char*>(plan_device);
  const GemmBatchProblem* probs = reinterpret_cast<const GemmBatchProblem*>(base + sizeof(GemmBatchHeader));
  const GemmTileRec* tiles = reinterpret_cast<const GemmTileRec*>(
      base + sizeof(GemmBatchHeader) + (size_t)h.count * sizeof(GemmBatchProblem));
  const GemmSplitTile* sts = reinterpret_cast<const GemmSplitTile*>(tiles + h.num_tiles);
  float* partials = static_cast<float*>(workspace);
  switch (h.bits) {
    case 2: launch_batched_bits<2>(probs, tiles, h, partials, st); break;
    case 3: launch_batched_bits<3>(probs, tiles, h, partials, st); break;
    case 4: launch_batched_bits<4>(probs, tiles, h, partials, st); break;
    case 5: launch_batched_bits<5>(probs, tiles, h, partials, st); break;
    case 6: launch_batched_bits<6>(probs, tiles, h, partials, st); break;
    case 8: launch_batched_bits<8>(probs, tiles, h, partials, st); break;
    case 16: launch_batched_bits<16>(probs, tiles, h, partials, st); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || h.splits == 1 || h.split_tiles == 0) return e;
  const int bn = h.nb * 128;
  const dim3 grid(h.split_tiles * (h.bm * bn / 1024));
  switch (h.splits) {
#define QMM_REDUCE_CASE(S) \
    case S: hipLaunchKernelGGL(qgemm_batched_reduce_kernel<S>, grid, dim3(256), 0, st, probs, sts, partials, h.bm, bn, S); break;
    QMM_REDUCE_CASE(2) QMM_REDUCE_CASE(3) QMM_REDUCE_CASE(4) QMM_REDUCE_CASE(5) QMM_REDUCE_CASE(6)
    QMM_REDUCE_CASE(8) QMM_REDUCE_CASE(10) QMM_REDUCE_CASE(12) QMM_REDUCE_CASE(16)
#undef QMM_REDUCE_CASE
    default:
      hipLaunchKernelGGL(qgemm_batched_reduce_kernel<0>, grid, dim3(256), 0, st, probs, sts, partials, h.bm, bn,
                         h.splits);
  }
  return hipGetLastError();
}

}  // namespace qmm

