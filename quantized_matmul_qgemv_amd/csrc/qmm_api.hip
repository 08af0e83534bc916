// C ABI of the library (declared in include/qmm.h): argument validation on
// the host, geometry choice, launch on the caller's stream, and a static
// thread-local error message (BaseRT, native-Metal LLM inference on Apple
// Silicon, §3.2: error handling through static thread-local buffers, no
// allocation on the hot path).  Validation never calls into HIP, so every
// error path runs without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qmm.h"
#include "qmm_internal.h"

namespace {

thread_local char g_err[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = '\0'; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return QMM_OK;
  return fail(QMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

#define CHECK_PTR(p, a)                                                                  \
  do {                                                                                   \
    if ((p) == nullptr) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer " #p, fn);    \
    if (!aligned((p), (a)))                                                              \
      return fail(QMM_ERR_INVALID_ARG, "%s: " #p " is not %d-byte aligned", fn, (int)(a)); \
  } while (0)

// Maximum k of the GEMV kernels: activations of one row are staged in LDS.
constexpr int kGemvMaxK = 16384;
constexpr int kMaxExperts = 1024;

// Quantized weights: 2, 3, 4, 5, 6 and 8 bits, groups of 32, 64 or 128.
// bits = 16 (unquantized fp16 weights) is accepted by the matmul entry
// points only (allow16); it has no scales, and group_size must still be
// one of the supported values (it is not used).
int check_format(const char* fn, int bits, int group_size, bool allow16 = false) {
  if (!(bits == 16 && allow16) && (bits < 2 || bits > 8 || bits == 7))
    return fail(QMM_ERR_UNSUPPORTED, "%s: bits=%d not supported (2, 3, 4, 5, 6 or 8%s)", fn, bits,
                allow16 ? "; 16 for fp16 weights" : "");
  if (group_size != 32 && group_size != 64 && group_size != 128)
    return fail(QMM_ERR_UNSUPPORTED, "%s: group_size=%d not supported (32, 64 or 128)", fn, group_size);
  return QMM_OK;
}



int check_nk(const char* fn, int n, int k, int group_size = 64) {
  if (n < 1) return fail(QMM_ERR_INVALID_ARG, "%s: n=%d must be >= 1", fn, n);
  if (k < 64 || k % 64 != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: k=%d must be a positive multiple of 64", fn, k);
  if (k % group_size != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: k=%d must be a multiple of group_size %d", fn, k, group_size);
  return QMM_OK;
}

// A routing plan must be at least as large as the one qmm_moe_route writes
// for (t, top_k, e); one built for other counts is also detected on the
// device (the output becomes NaN), but a buffer too small for these counts
// would be read past its end, so it is refused here.
int check_plan_size(const char* fn, size_t plan_bytes, int t, int top_k, int e) {
  const size_t need = qmm::grouped_workspace_bytes(t, top_k, e, 0);
  if (plan_bytes < need)
    return fail(QMM_ERR_WORKSPACE, "%s: plan of %zu bytes, a routing plan for t=%d top_k=%d e=%d has %zu",
                fn, plan_bytes, t, top_k, e, need);
  return QMM_OK;
}

}  // namespace

extern "C" {

int qmm_version(void) { return 100; }

const char* qmm_last_error(void) { return g_err; }

int qmm_qgemv(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
              const uint16_t* x, float* y, int n, int k, int bits, int group_size,
              qmm_stream stream) {
  const char* fn = "qmm_qgemv";
  clear_error();
  if (int st = check_format(fn, bits, group_size, true)) return st;
  if (int st = check_nk(fn, n, k, group_size)) return st;
  if (k > kGemvMaxK) return fail(QMM_ERR_INVALID_ARG, "%s: k=%d exceeds %d", fn, k, kGemvMaxK);
  CHECK_PTR(w, 16);
  if (bits != 16) {  // fp16 weights have no scales or biases
    CHECK_PTR(scales, 2);
    CHECK_PTR(biases, 2);
  }
  CHECK_PTR(x, 16);
  CHECK_PTR(y, 4);
  qmm::GemvProblem p{w, scales, biases, x, y, n, k};
  const qmm::GemvGeom g = qmm::gemv_choose(n, k, bits);
  return hip_status(qmm::launch_qgemv(p, bits, group_size, g, (hipStream_t)stream), fn);
}

int qmm_qgemv_batched_plan(const qmm_gemv_problem* problems, int count, int bits,
                           int group_size, void* plan, size_t plan_bytes,
                           size_t* plan_bytes_needed) {
  const char* fn = "qmm_qgemv_batched_plan";
  clear_error();
  if (int st = check_format(fn, bits, group_size, true)) return st;
  if (count < 1) return fail(QMM_ERR_INVALID_ARG, "%s: count=%d must be >= 1", fn, count);
  if (problems == nullptr) return fail(QMM_ERR_INVALID_ARG, "%s: null problems", fn);
  int lpr = 16, max_groups = 0;
  for (int i = 0; i < count; ++i) {
    const qmm_gemv_problem& q = problems[i];
    if (check_nk(fn, q.n, q.k, group_size)) return fail(QMM_ERR_INVALID_ARG, "%s: problem %d: n=%d k=%d invalid", fn, i, q.n, q.k);
    if (q.k > kGemvMaxK) return fail(QMM_ERR_INVALID_ARG, "%s: problem %d: k=%d exceeds %d", fn, i, q.k, kGemvMaxK);
    if (!q.w || (bits != 16 && (!q.scales || !q.biases)) || !q.x || !q.y)
      return fail(QMM_ERR_INVALID_ARG, "%s: problem %d has a null pointer", fn, i);
    if (!aligned(q.w, 16) || !aligned(q.x, 16) || !aligned(q.y, 4) || !aligned(q.scales, 2) ||
        !aligned(q.biases, 2))
      return fail(QMM_ERR_INVALID_ARG, "%s: problem %d has a misaligned pointer", fn, i);
    const int groups = q.k / 64;
    const int l = qmm::gemv_lanes_for_groups(groups);
    if (l < lpr) lpr = l;
    if (groups > max_groups) max_groups = groups;
  }
  const int rows = qmm::gemv_rows_per_pass(lpr, qmm::gemv_row_unroll(bits), 1);
  // Passes per workgroup.  One pass per workgroup measured best on the decode
  // sweeps: the hardware dispatcher then balances thousands of short
  // workgroups across the CUs, where longer multi-pass workgroups leave a
  // tail.  QMM_GEMV_TARGET_BLOCKS sets a workgroup target instead (tuning
  // sweeps), weighting each pass by its k.
  double target = 1e12;
  if (const char* env = getenv("QMM_GEMV_TARGET_BLOCKS")) {
    const double v = atof(env);
    if (v >= 1.0) target = v;
  }
  double units = 0.0;
  for (int i = 0; i < count; ++i)
    units += (double)((problems[i].n + rows - 1) / rows) * problems[i].k / 1024.0;
  const double base = units / target < 1.0 ? 1.0 : units / target;
  auto passes_of = [&](int k) {
    const int p = (int)(base * 1024.0 / k + 0.5);
    return p < 1 ? 1 : (p > 16 ? 16 : p);
  };
  long blocks = 0;
  for (int i = 0; i < count; ++i) {
    const int chunk = rows * passes_of(problems[i].k);
    blocks += (problems[i].n + chunk - 1) / chunk;
  }
  if (blocks > 0x7FFFFFFFL) return fail(QMM_ERR_INVALID_ARG, "%s: too many blocks", fn);
  const size_t need = sizeof(qmm::GemvPlanHeader) + (size_t)blocks * sizeof(qmm::GemvBlock);
  if (plan_bytes_needed) *plan_bytes_needed = need;
  if (plan == nullptr || plan_bytes < need)
    return fail(QMM_ERR_WORKSPACE, "%s: plan buffer of %zu bytes, %zu needed", fn, plan_bytes, need);
  if (!aligned(plan, 8)) return fail(QMM_ERR_INVALID_ARG, "%s: plan is not 8-byte aligned", fn);
  qmm::GemvPlanHeader hdr;
  memset(&hdr, 0, sizeof hdr);
  hdr.magic = qmm::kPlanMagic;
  hdr.version = qmm::kPlanVersion;
  hdr.bits = bits;
  hdr.group_size = group_size;
  hdr.lanes_per_row = lpr;
  hdr.rows_per_block = rows;
  hdr.num_blocks = (int32_t)blocks;
  hdr.max_groups = max_groups;
  hdr.count = count;
  // The caller's buffer is only 8-byte aligned, so the 64-byte-aligned
  // records are copied in byte-wise rather than stored as structures.
  unsigned char* out = static_cast<unsigned char*>(plan);
  memcpy(out, &hdr, sizeof hdr);
  unsigned char* recs = out + sizeof hdr;
  long bi = 0;
  for (int i = 0; i < count; ++i) {
    const qmm_gemv_problem& q = problems[i];
    const int chunk = rows * passes_of(q.k);
    for (int r = 0; r < q.n; r += chunk) {
      qmm::GemvBlock blk;
      memset(&blk, 0, sizeof blk);
      blk.p = qmm::GemvProblem{q.w, q.scales, q.biases, q.x, q.y, q.n, q.k};
      blk.row0 = r;
      blk.nrows = q.n - r < chunk ? q.n - r : chunk;
      memcpy(recs + (size_t)bi++ * sizeof blk, &blk, sizeof blk);
    }
  }
  return QMM_OK;
}

int qmm_qgemv_batched(const void* plan_device, const void* plan_host, qmm_stream stream) {
  const char* fn = "qmm_qgemv_batched";
  clear_error();
  if (plan_host == nullptr) return fail(QMM_ERR_INVALID_ARG, "%s: null plan_host", fn);
  CHECK_PTR(plan_device, 64);
  qmm::GemvPlanHeader hdr;
  memcpy(&hdr, plan_host, sizeof hdr);
  if (hdr.magic != qmm::kPlanMagic || hdr.version != qmm::kPlanVersion)
    return fail(QMM_ERR_INVALID_ARG, "%s: plan_host is not a plan image", fn);
  if (int st = check_format(fn, hdr.bits, hdr.group_size, true)) return st;
  if (hdr.num_blocks < 1 || hdr.max_groups < 1 || hdr.max_groups > kGemvMaxK / 64)
    return fail(QMM_ERR_INVALID_ARG, "%s: corrupt plan header", fn);
  const qmm::GemvBlock* recs = reinterpret_cast<const qmm::GemvBlock*>(
      static_cast<const unsigned char*>(plan_device) + sizeof(qmm::GemvPlanHeader));
  return hip_status(qmm::launch_qgemv_batched(recs, hdr.num_blocks, hdr.bits, hdr.group_size, hdr.lanes_per_row,
                                              hdr.max_groups, (hipStream_t)stream),
                    fn);
}

// Scale layout flag of the GEMM entry points: interleaved scales need
// tile-interleaved weights, groups of 64, quantized codes and k % 256 == 0.
static int check_stiled(const char* fn, int stiled, int wtiled, int bits, int group_size, int k) {
  if (!stiled) return QMM_OK;
  if (!wtiled) return fail(QMM_ERR_INVALID_ARG, "%s: QMM_SCALES_TILED needs QMM_WEIGHTS_TILED", fn);
  if (bits == 16) return fail(QMM_ERR_INVALID_ARG, "%s: fp16 weights have no scales to interleave", fn);
  if (group_size != 64 || k % 256 != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: interleaved scales need group_size 64 and k %% 256 == 0 (k=%d)", fn, k);
  return QMM_OK;
}

size_t qmm_qgemm_workspace_size(int m, int n, int k, int bits, int group_size) {
  bits &= ~(QMM_WEIGHTS_TILED | QMM_SCALES_TILED);  // the layouts do not change the split-k workspace
  if (m < 1 || n < 1 || k < 64 || k % 64 != 0) return 0;
  if ((group_size != 32 && group_size != 64 && group_size != 128) || k % group_size != 0) return 0;
  if ((bits < 2 || bits > 8 || bits == 7) && bits != 16) return 0;
  return qmm::gemm_workspace_bytes(m, n, k, bits);
}

int qmm_qgemm(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
              const uint16_t* x, float* y, int m, int n, int k, int bits, int group_size,
              void* workspace, size_t workspace_bytes, qmm_stream stream) {
  const char* fn = "qmm_qgemm";
  clear_error();
  const int wtiled = (bits & QMM_WEIGHTS_TILED) ? 1 : 0;
  const int stiled = (bits & QMM_SCALES_TILED) ? 1 : 0;
  bits &= ~(QMM_WEIGHTS_TILED | QMM_SCALES_TILED);
  if (int st = check_format(fn, bits, group_size, true)) return st;
  if (m < 0) return fail(QMM_ERR_INVALID_ARG, "%s: m=%d must be >= 0", fn, m);
  if (int st = check_nk(fn, n, k, group_size)) return st;
  if (wtiled && n % 32 != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: n=%d must be a multiple of 32 for tile-interleaved weights", fn, n);
  if (int st = check_stiled(fn, stiled, wtiled, bits, group_size, k)) return st;
  if (m == 0) return QMM_OK;
  CHECK_PTR(w, 16);
  if (stiled) {  // one interleaved array holds the scales and the biases
    CHECK_PTR(scales, 16);
  } else if (bits != 16) {  // fp16 weights have no scales or biases
    CHECK_PTR(scales, 2);
    CHECK_PTR(biases, 2);
  }
  CHECK_PTR(x, 16);
  CHECK_PTR(y, 4);
  const size_t need = qmm::gemm_workspace_bytes(m, n, k, bits);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(QMM_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    CHECK_PTR(workspace, 16);
  }
  qmm::GemmArgs a{w, scales, stiled ? nullptr : biases, x, y, m, n, k, group_size, wtiled, stiled};
  return hip_status(qmm::launch_qgemm(a, bits, workspace, (hipStream_t)stream), fn);
}

int qmm_qgemm_batched_plan(const qmm_gemm_problem* problems, int count, int bits,
                           int group_size, void* plan, size_t plan_bytes,
                           size_t* plan_bytes_needed, size_t* workspace_bytes_needed) {
  const char* fn = "qmm_qgemm_batched_plan";
  clear_error();
  const int wtiled = (bits & QMM_WEIGHTS_TILED) ? 1 : 0;
  const int stiled = (bits & QMM_SCALES_TILED) ? 1 : 0;
  bits &= ~(QMM_WEIGHTS_TILED | QMM_SCALES_TILED);
  if (int st = check_format(fn, bits, group_size, true)) return st;
  if (stiled && !wtiled) return fail(QMM_ERR_INVALID_ARG, "%s: QMM_SCALES_TILED needs QMM_WEIGHTS_TILED", fn);
  if (stiled && (bits == 16 || group_size != 64))
    return fail(QMM_ERR_INVALID_ARG, "%s: interleaved scales need quantized codes and group_size 64", fn);
  if (count < 1) return fail(QMM_ERR_INVALID_ARG, "%s: count=%d must be >= 1", fn, count);
  if (count > (1 << 20)) return fail(QMM_ERR_INVALID_ARG, "%s: count=%d too large", fn, count);
  if (problems == nullptr) return fail(QMM_ERR_INVALID_ARG, "%s: null problems", fn);
  // GemmBatchProblem is 64-byte aligned (one device cache line per record);
  // calloc guarantees only 16, so the host copy is allocated aligned.
  const size_t probs_bytes = (size_t)count * sizeof(qmm::GemmBatchProblem);
  qmm::GemmBatchProblem* probs =
      static_cast<qmm::GemmBatchProblem*>(aligned_alloc(alignof(qmm::GemmBatchProblem), probs_bytes));
  if (probs == nullptr) return fail(QMM_ERR_INVALID_ARG, "%s: out of host memory", fn);
  memset(probs, 0, probs_bytes);
  for (int i = 0; i < count; ++i) {
    const qmm_gemm_problem& q = problems[i];
    int bad = 0;
    // an empty problem (m = 0) is never read or written: x and y may be null
    if (q.m < 0 || check_nk(fn, q.n, q.k, group_size) || (wtiled && q.n % 32 != 0) ||
        (stiled && q.k % 256 != 0)) bad = 1;
    else if (!q.w || (bits != 16 && (!q.scales || (!stiled && !q.biases))) || (q.m > 0 && (!q.x || !q.y))) bad = 2;
    else if (!aligned(q.w, 16) || !aligned(q.x, 16) || !aligned(q.y, 4) ||
             !aligned(q.scales, stiled ? 16 : 2) || (!stiled && !aligned(q.biases, 2))) bad = 3;
    if (bad) {
      free(probs);
      return fail(QMM_ERR_INVALID_ARG, "%s: problem %d: %s", fn, i,
                  bad == 1 ? (stiled ? "bad m, n or k (interleaved scales need n % 32 == 0 and k % 256 == 0)"
                              : wtiled ? "bad m, n or k (tile-interleaved weights need n % 32 == 0)"
                                       : "bad m, n or k")
                           : bad == 2 ? "null pointer" : "misaligned pointer");
    }
    probs[i].w = q.w;
    probs[i].s = q.scales;
    probs[i].b = stiled ? nullptr : q.biases;
    probs[i].x = q.x;
    probs[i].y = q.y;
    probs[i].m = q.m;
    probs[i].n = q.n;
    probs[i].k = q.k;
  }
  const size_t need = qmm::gemm_batch_build(probs, count, bits, group_size, wtiled, stiled, nullptr, 0);
  if (plan_bytes_needed) *plan_bytes_needed = need;
  if (plan == nullptr || plan_bytes < need) {
    free(probs);
    return fail(QMM_ERR_WORKSPACE, "%s: plan buffer of %zu bytes, %zu needed", fn, plan_bytes, need);
  }
  if (!aligned(plan, 8)) {
    free(probs);
    return fail(QMM_ERR_INVALID_ARG, "%s: plan is not 8-byte aligned", fn);
  }
  qmm::gemm_batch_build(probs, count, bits, group_size, wtiled, stiled, plan, plan_bytes);
  free(probs);
  qmm::GemmBatchHeader hdr;
  memcpy(&hdr, plan, sizeof hdr);
  if (workspace_bytes_needed) *workspace_bytes_needed = (size_t)hdr.workspace_bytes;
  return QMM_OK;
}

int qmm_qgemm_batched(const void* plan_device, const void* plan_host, void* workspace,
                      size_t workspace_bytes, qmm_stream stream) {
  const char* fn = "qmm_qgemm_batched";
  clear_error();
  if (plan_host == nullptr) return fail(QMM_ERR_INVALID_ARG, "%s: null plan_host", fn);
  CHECK_PTR(plan_device, 16);
  qmm::GemmBatchHeader hdr;
  memcpy(&hdr, plan_host, sizeof hdr);
  if (hdr.magic != qmm::kBatchMagic || hdr.version != qmm::kBatchVersion)
    return fail(QMM_ERR_INVALID_ARG, "%s: plan_host is not a batched-GEMM plan image", fn);
  if (int st = check_format(fn, hdr.bits, hdr.group_size, true)) return st;
  if (hdr.count < 1 || hdr.num_tiles < 0 || hdr.splits < 1 || (hdr.wtiled != 0 && hdr.wtiled != 1) ||
      (hdr.stiled != 0 && hdr.stiled != 1) || (hdr.stiled == 1 && (hdr.wtiled != 1 || hdr.group_size != 64)) ||
      !(hdr.bm == 32 || hdr.bm == 64 || hdr.bm == 128 || hdr.bm == 256) ||
      !(hdr.nb == 1 || hdr.nb == 2) || (hdr.bm == 256 && hdr.nb != 2) || (hdr.bits == 16 && hdr.nb != 1) ||
      !(hdr.kw == 1 || hdr.kw == 2) || (hdr.kw == 2 && (hdr.bm == 256 || (hdr.nb == 2 && hdr.bm != 64))))
    return fail(QMM_ERR_INVALID_ARG, "%s: corrupt plan header", fn);
  if (hdr.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < hdr.workspace_bytes)
      return fail(QMM_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                  (size_t)hdr.workspace_bytes);
    CHECK_PTR(workspace, 16);
  }
  if (hdr.num_tiles == 0) return QMM_OK;
  return hip_status(qmm::launch_qgemm_batched(plan_device, hdr, workspace, (hipStream_t)stream), fn);
}

size_t qmm_qgemm_grouped_workspace_size(int t, int top_k, int e, int n, int k, int bits,
                                        int group_size) {
  (void)k; (void)bits; (void)group_size;
  if (t < 0 || top_k < 1 || e < 1) return 0;
  return qmm::grouped_workspace_bytes(t, top_k, e, n);
}

int qmm_qgemm_grouped(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                      const uint16_t* a, int a_row_per_pair, const int32_t* expert_ids,
                      float* y, int t, int top_k, int e, int n, int k, int bits,
                      int group_size, void* workspace, size_t workspace_bytes,
                      qmm_stream stream) {
  const char* fn = "qmm_qgemm_grouped";
  clear_error();
  const int wtiled = (bits & QMM_WEIGHTS_TILED) ? 1 : 0;
  const int stiled = (bits & QMM_SCALES_TILED) ? 1 : 0;
  bits &= ~(QMM_WEIGHTS_TILED | QMM_SCALES_TILED);
  if (int st = check_format(fn, bits, group_size, true)) return st;
  if (t < 0) return fail(QMM_ERR_INVALID_ARG, "%s: t=%d must be >= 0", fn, t);
  if (top_k < 1) return fail(QMM_ERR_INVALID_ARG, "%s: top_k=%d must be >= 1", fn, top_k);
  if (e < 1 || e > kMaxExperts)
    return fail(QMM_ERR_INVALID_ARG, "%s: e=%d must be in [1, %d]", fn, e, kMaxExperts);
  if (a_row_per_pair != 0 && a_row_per_pair != 1)
    return fail(QMM_ERR_INVALID_ARG, "%s: a_row_per_pair must be 0 or 1", fn);
  if (int st = check_nk(fn, n, k, group_size)) return st;
  if (wtiled && n % 32 != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: n=%d must be a multiple of 32 for tile-interleaved weights", fn, n);
  if (int st = check_stiled(fn, stiled, wtiled, bits, group_size, k)) return st;
  if ((long)t * top_k > 0x7FFFFFFFL / 4) return fail(QMM_ERR_INVALID_ARG, "%s: too many pairs", fn);
  if (t == 0) return QMM_OK;
  CHECK_PTR(w, 16);
  if (stiled) {  // one interleaved array holds the scales and the biases
    CHECK_PTR(scales, 16);
  } else if (bits != 16) {  // fp16 weights have no scales or biases
    CHECK_PTR(scales, 2);
    CHECK_PTR(biases, 2);
  }
  CHECK_PTR(a, 16);
  CHECK_PTR(expert_ids, 4);
  CHECK_PTR(y, 4);
  const size_t need = qmm::grouped_workspace_bytes(t, top_k, e, n);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(QMM_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  CHECK_PTR(workspace, 16);
  qmm::GroupedArgs ga{w, scales, stiled ? nullptr : biases, a, a_row_per_pair, expert_ids, y, t, top_k, e, n, k, group_size, wtiled, stiled};
  return hip_status(qmm::launch_qgemm_grouped(ga, bits, workspace, true, (hipStream_t)stream), fn);
}

int qmm_qgemm_grouped_noalloc(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                              const uint16_t* a, int a_row_per_pair, const int32_t* expert_ids,
                              float* y, int t, int top_k, int e, int n, int k, int bits,
                              int group_size, qmm_stream stream) {
  const char* fn = "qmm_qgemm_grouped_noalloc";
  clear_error();
  const int wtiled = (bits & QMM_WEIGHTS_TILED) ? 1 : 0;
  const int stiled = (bits & QMM_SCALES_TILED) ? 1 : 0;
  bits &= ~(QMM_WEIGHTS_TILED | QMM_SCALES_TILED);
  if (int st = check_format(fn, bits, group_size, true)) return st;
  if (t < 0) return fail(QMM_ERR_INVALID_ARG, "%s: t=%d must be >= 0", fn, t);
  if (top_k < 1) return fail(QMM_ERR_INVALID_ARG, "%s: top_k=%d must be >= 1", fn, top_k);
  if (e < 1 || e > kMaxExperts)
    return fail(QMM_ERR_INVALID_ARG, "%s: e=%d must be in [1, %d]", fn, e, kMaxExperts);
  if (a_row_per_pair != 0 && a_row_per_pair != 1)
    return fail(QMM_ERR_INVALID_ARG, "%s: a_row_per_pair must be 0 or 1", fn);
  if (int st = check_nk(fn, n, k, group_size)) return st;
  if (wtiled && n % 32 != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: n=%d must be a multiple of 32 for tile-interleaved weights", fn, n);
  if (int st = check_stiled(fn, stiled, wtiled, bits, group_size, k)) return st;
  if ((long)t * top_k > 0x7FFFFFFFL / 4) return fail(QMM_ERR_INVALID_ARG, "%s: too many pairs", fn);
  if (t == 0) return QMM_OK;
  CHECK_PTR(w, 16);
  if (stiled) {  // one interleaved array holds the scales and the biases
    CHECK_PTR(scales, 16);
  } else if (bits != 16) {  // fp16 weights have no scales or biases
    CHECK_PTR(scales, 2);
    CHECK_PTR(biases, 2);
  }
  CHECK_PTR(a, 16);
  CHECK_PTR(expert_ids, 4);
  CHECK_PTR(y, 4);
  const size_t need = qmm::grouped_workspace_bytes(t, top_k, e, n);
  if (need > qmm::kGroupedScratchBytes)
    return fail(QMM_ERR_WORKSPACE,
                "%s: t=%d top_k=%d e=%d needs %zu bytes of scratch; the static scratch holds %zu "
                "(use qmm_qgemm_grouped with a workspace)",
                fn, t, top_k, e, need, qmm::kGroupedScratchBytes);
  void* scratch = nullptr;
  if (int st = hip_status(qmm::grouped_scratch(&scratch), fn)) return st;
  qmm::GroupedArgs ga{w, scales, stiled ? nullptr : biases, a, a_row_per_pair, expert_ids, y, t, top_k, e, n, k, group_size, wtiled, stiled};
  return hip_status(qmm::launch_qgemm_grouped(ga, bits, scratch, true, (hipStream_t)stream), fn);
}

size_t qmm_moe_route_size(int t, int top_k, int e) {
  if (t < 0 || top_k < 1 || e < 1 || e > kMaxExperts) return 0;
  if ((long)t * top_k > 0x7FFFFFFFL / 4) return 0;
  return qmm::grouped_workspace_bytes(t, top_k, e, 0);
}

int qmm_moe_route(const int32_t* expert_ids, int t, int top_k, int e, void* plan,
                  size_t plan_bytes, qmm_stream stream) {
  const char* fn = "qmm_moe_route";
  clear_error();
  if (t < 0) return fail(QMM_ERR_INVALID_ARG, "%s: t=%d must be >= 0", fn, t);
  if (top_k < 1) return fail(QMM_ERR_INVALID_ARG, "%s: top_k=%d must be >= 1", fn, top_k);
  if (e < 1 || e > kMaxExperts)
    return fail(QMM_ERR_INVALID_ARG, "%s: e=%d must be in [1, %d]", fn, e, kMaxExperts);
  if ((long)t * top_k > 0x7FFFFFFFL / 4) return fail(QMM_ERR_INVALID_ARG, "%s: too many pairs", fn);
  if (t == 0) return QMM_OK;
  CHECK_PTR(expert_ids, 4);
  const size_t need = qmm::grouped_workspace_bytes(t, top_k, e, 0);
  if (plan == nullptr || plan_bytes < need)
    return fail(QMM_ERR_WORKSPACE, "%s: plan of %zu bytes, %zu needed", fn, plan_bytes, need);
  CHECK_PTR(plan, 16);
  return hip_status(qmm::launch_moe_route(expert_ids, t, top_k, e, plan, (hipStream_t)stream), fn);
}

int qmm_qgemm_grouped_routed(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                             const uint16_t* a, int a_row_per_pair, const void* plan,
                             size_t plan_bytes, float* y, int t, int top_k, int e, int n, int k,
                             int bits, int group_size, qmm_stream stream) {
  const char* fn = "qmm_qgemm_grouped_routed";
  clear_error();
  const int wtiled = (bits & QMM_WEIGHTS_TILED) ? 1 : 0;
  const int stiled = (bits & QMM_SCALES_TILED) ? 1 : 0;
  bits &= ~(QMM_WEIGHTS_TILED | QMM_SCALES_TILED);
  if (int st = check_format(fn, bits, group_size, true)) return st;
  if (t < 0) return fail(QMM_ERR_INVALID_ARG, "%s: t=%d must be >= 0", fn, t);
  if (top_k < 1) return fail(QMM_ERR_INVALID_ARG, "%s: top_k=%d must be >= 1", fn, top_k);
  if (e < 1 || e > kMaxExperts)
    return fail(QMM_ERR_INVALID_ARG, "%s: e=%d must be in [1, %d]", fn, e, kMaxExperts);
  if (a_row_per_pair != 0 && a_row_per_pair != 1)
    return fail(QMM_ERR_INVALID_ARG, "%s: a_row_per_pair must be 0 or 1", fn);
  if (int st = check_nk(fn, n, k, group_size)) return st;
  if (wtiled && n % 32 != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: n=%d must be a multiple of 32 for tile-interleaved weights", fn, n);
  if (int st = check_stiled(fn, stiled, wtiled, bits, group_size, k)) return st;
  if ((long)t * top_k > 0x7FFFFFFFL / 4) return fail(QMM_ERR_INVALID_ARG, "%s: too many pairs", fn);
  if (t == 0) return QMM_OK;
  CHECK_PTR(w, 16);
  if (stiled) {  // one interleaved array holds the scales and the biases
    CHECK_PTR(scales, 16);
  } else if (bits != 16) {  // fp16 weights have no scales or biases
    CHECK_PTR(scales, 2);
    CHECK_PTR(biases, 2);
  }
  CHECK_PTR(a, 16);
  CHECK_PTR(plan, 16);
  CHECK_PTR(y, 4);
  if (int st = check_plan_size(fn, plan_bytes, t, top_k, e)) return st;
  qmm::GroupedArgs ga{w, scales, stiled ? nullptr : biases, a, a_row_per_pair, nullptr, y, t, top_k, e, n, k, group_size, wtiled, stiled};
  return hip_status(qmm::launch_qgemm_grouped(ga, bits, const_cast<void*>(plan), false,
                                              (hipStream_t)stream), fn);
}

int qmm_moe_gate_up_swiglu(const uint32_t* w_gate, const uint16_t* s_gate, const uint16_t* b_gate,
                           const uint32_t* w_up, const uint16_t* s_up, const uint16_t* b_up,
                           const uint16_t* x, const void* plan, size_t plan_bytes, uint16_t* h,
                           int t, int top_k, int e, int n, int k, int bits, int group_size,
                           qmm_stream stream) {
  const char* fn = "qmm_moe_gate_up_swiglu";
  clear_error();
  const int wtiled = (bits & QMM_WEIGHTS_TILED) ? 1 : 0;
  const int stiled = (bits & QMM_SCALES_TILED) ? 1 : 0;
  bits &= ~(QMM_WEIGHTS_TILED | QMM_SCALES_TILED);
  if (int st = check_format(fn, bits, group_size, true)) return st;
  if (t < 0) return fail(QMM_ERR_INVALID_ARG, "%s: t=%d must be >= 0", fn, t);
  if (top_k < 1) return fail(QMM_ERR_INVALID_ARG, "%s: top_k=%d must be >= 1", fn, top_k);
  if (e < 1 || e > kMaxExperts)
    return fail(QMM_ERR_INVALID_ARG, "%s: e=%d must be in [1, %d]", fn, e, kMaxExperts);
  if (int st = check_nk(fn, n, k, group_size)) return st;
  if (wtiled && n % 32 != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: n=%d must be a multiple of 32 for tile-interleaved weights", fn, n);
  if (int st = check_stiled(fn, stiled, wtiled, bits, group_size, k)) return st;
  if ((long)t * top_k > 0x7FFFFFFFL / 4) return fail(QMM_ERR_INVALID_ARG, "%s: too many pairs", fn);
  if (t == 0) return QMM_OK;
  CHECK_PTR(w_gate, 16);
  CHECK_PTR(w_up, 16);
  if (stiled) {  // interleaved arrays hold the scales and the biases
    CHECK_PTR(s_gate, 16);
    CHECK_PTR(s_up, 16);
  } else if (bits != 16) {
    CHECK_PTR(s_gate, 2);
    CHECK_PTR(b_gate, 2);
    CHECK_PTR(s_up, 2);
    CHECK_PTR(b_up, 2);
  }
  CHECK_PTR(x, 16);
  CHECK_PTR(plan, 16);
  CHECK_PTR(h, 2);
  if (int st = check_plan_size(fn, plan_bytes, t, top_k, e)) return st;
  return hip_status(qmm::launch_moe_swiglu(w_gate, s_gate, stiled ? nullptr : b_gate, w_up, s_up,
                                           stiled ? nullptr : b_up, x, plan, h, t, top_k, e, n, k, bits,
                                           group_size, wtiled, stiled, (hipStream_t)stream),
                    fn);
}

int qmm_moe_combine(const float* y_pairs, const float* weights, float* y, int t, int top_k, int n,
                    qmm_stream stream) {
  const char* fn = "qmm_moe_combine";
  clear_error();
  if (t < 0) return fail(QMM_ERR_INVALID_ARG, "%s: t=%d must be >= 0", fn, t);
  if (top_k < 1) return fail(QMM_ERR_INVALID_ARG, "%s: top_k=%d must be >= 1", fn, top_k);
  if (n < 1) return fail(QMM_ERR_INVALID_ARG, "%s: n=%d must be >= 1", fn, n);
  if ((long)t * top_k * n > 0x7FFFFFFFFFL) return fail(QMM_ERR_INVALID_ARG, "%s: too large", fn);
  if (t == 0) return QMM_OK;
  CHECK_PTR(y_pairs, 4);
  CHECK_PTR(weights, 4);
  CHECK_PTR(y, 4);
  return hip_status(qmm::launch_moe_combine(y_pairs, weights, y, t, top_k, n, (hipStream_t)stream), fn);
}

int qmm_quantize(const float* w_f32, uint32_t* words, uint16_t* scales, uint16_t* biases,
                 int n, int k, int bits, int group_size, qmm_stream stream) {
  const char* fn = "qmm_quantize";
  clear_error();
  if (int st = check_format(fn, bits, group_size)) return st;
  if (int st = check_nk(fn, n, k, group_size)) return st;
  CHECK_PTR(w_f32, 16);
  CHECK_PTR(words, 4);
  CHECK_PTR(scales, 2);
  CHECK_PTR(biases, 2);
  return hip_status(qmm::launch_quantize(w_f32, words, scales, biases, n, k, bits, group_size, (hipStream_t)stream), fn);
}

int qmm_convert_bf16(const uint16_t* src, uint16_t* dst, size_t count, qmm_stream stream) {
  const char* fn = "qmm_convert_bf16";
  clear_error();
  if (count == 0) return QMM_OK;
  if (count % 2 != 0) return fail(QMM_ERR_INVALID_ARG, "%s: count=%zu must be even", fn, count);
  if (count > ((size_t)1 << 40)) return fail(QMM_ERR_INVALID_ARG, "%s: count=%zu too large", fn, count);
  CHECK_PTR(src, 4);
  CHECK_PTR(dst, 4);
  return hip_status(qmm::launch_convert_bf16(src, dst, (long)count, (hipStream_t)stream), fn);
}

int qmm_repack_tiled(const uint32_t* w, uint32_t* out, int n, int k, int bits, qmm_stream stream) {
  const char* fn = "qmm_repack_tiled";
  clear_error();
  if (int st = check_format(fn, bits, 64, true)) return st;
  if (int st = check_nk(fn, n, k)) return st;
  if (n % 32 != 0) return fail(QMM_ERR_INVALID_ARG, "%s: n=%d must be a multiple of 32", fn, n);
  CHECK_PTR(w, 16);
  CHECK_PTR(out, 16);
  const size_t bytes = (size_t)n * (size_t)(k / 64) * (size_t)bits * 8;
  const uintptr_t a = (uintptr_t)w, b = (uintptr_t)out;
  if (a < b + bytes && b < a + bytes) return fail(QMM_ERR_INVALID_ARG, "%s: w and out overlap", fn);
  return hip_status(qmm::launch_repack_tiled(w, out, n, k, bits, (hipStream_t)stream), fn);
}

int qmm_repack_scales_tiled(const uint16_t* scales, const uint16_t* biases, uint16_t* out, int n, int k,
                            qmm_stream stream) {
  const char* fn = "qmm_repack_scales_tiled";
  clear_error();
  if (int st = check_nk(fn, n, k)) return st;
  if (n % 32 != 0) return fail(QMM_ERR_INVALID_ARG, "%s: n=%d must be a multiple of 32", fn, n);
  if (k % 256 != 0) return fail(QMM_ERR_INVALID_ARG, "%s: k=%d must be a multiple of 256", fn, k);
  CHECK_PTR(scales, 2);
  CHECK_PTR(biases, 2);
  CHECK_PTR(out, 16);
  const size_t half = (size_t)n * (size_t)(k / 64) * 2;  // bytes of scales (and of biases)
  const uintptr_t o = (uintptr_t)out, sp = (uintptr_t)scales, bp = (uintptr_t)biases;
  if ((o < sp + half && sp < o + 2 * half) || (o < bp + half && bp < o + 2 * half))
    return fail(QMM_ERR_INVALID_ARG, "%s: out overlaps scales or biases", fn);
  return hip_status(qmm::launch_repack_scales_tiled(scales, biases, out, n, k, (hipStream_t)stream), fn);
}

int qmm_unpack_codes(const uint32_t* w, uint8_t* codes, int n, int k, int bits,
                     qmm_stream stream) {
  const char* fn = "qmm_unpack_codes";
  clear_error();
  if (int st = check_format(fn, bits, 64)) return st;
  if (int st = check_nk(fn, n, k)) return st;
  CHECK_PTR(w, 4);
  CHECK_PTR(codes, 1);
  return hip_status(qmm::launch_unpack_codes(w, codes, n, k, bits, (hipStream_t)stream), fn);
}

int qmm_dequant(const uint32_t* w, const uint16_t* scales, const uint16_t* biases, void* out,
                int out_is_f16, int n, int k, int bits, int group_size, qmm_stream stream) {
  const char* fn = "qmm_dequant";
  clear_error();
  if (int st = check_format(fn, bits, group_size)) return st;
  if (int st = check_nk(fn, n, k, group_size)) return st;
  if (out_is_f16 != 0 && out_is_f16 != 1)
    return fail(QMM_ERR_INVALID_ARG, "%s: out_is_f16 must be 0 or 1", fn);
  CHECK_PTR(w, 4);
  CHECK_PTR(scales, 2);
  CHECK_PTR(biases, 2);
  CHECK_PTR(out, 4);
  return hip_status(qmm::launch_dequant(w, scales, biases, out, out_is_f16, n, k, bits, group_size, (hipStream_t)stream), fn);
}

}  // extern "C"
