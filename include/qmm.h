/*
 * qmm.h - C ABI of the MI355X (gfx950) weight-quantized GEMV / GEMM library.
 *
 * What the library computes
 * -------------------------
 * BaseRT (native-Metal LLM inference on Apple Silicon), §3.3 "kernel fusion
 * and specialization": matrix multiplies over group-quantized weights, one
 * GEMV variant for decode (M = 1) and one GEMM variant for prefill (M > 1),
 * with dequantization folded into the inner loop so that dequantized
 * weights never reach memory.  §3.4 "prefill": the M > 1 case is a tiled
 * GEMM on [seq_len x dim] activations and is compute-bound.  The abstract
 * and Fig. 1 add mixture-of-experts prefill (Qwen3-30B-A3B), served here by
 * a grouped GEMM over token-to-expert buckets.  §3 states that the runtime
 * is reached through a C API, and §3.2 that the decode loop allocates
 * nothing and reports errors through static thread-local buffers; this ABI
 * follows both.
 *
 * For every entry point, with W_hat[n, k] = s[n, k/gs] * q[n, k] + b[n, k/gs]:
 *     y[m, n] = sum_k x[m, k] * W_hat[n, k]          (fp32 accumulation)
 *
 * Data formats (all little-endian, all row-major)
 * ----------------------------------------------
 *   weights  W[n, k] is [out, in].  Codes q in 0 .. 2^bits - 1 are packed
 *            along k as a little-endian bit stream: code k occupies bits
 *            [bits*k, bits*k + bits) of its row, bit i of the stream is bit
 *            i % 32 of uint32 word i / 32.  For bits = 4 that is 8 nibbles per
 *            word, low nibble first; for bits = 8, 4 bytes per word, low byte
 *            first; 3-, 5- and 6-bit codes straddle word boundaries (every 8
 *            codes fill exactly `bits` bytes).  Row stride: k * bits / 32
 *            words; a 64-code group is 8 * bits bytes.  The GEMM entry points
 *            also read a tile-interleaved copy of these words (see
 *            qmm_repack_tiled and QMM_WEIGHTS_TILED).
 *   scales,  fp16 bit patterns (uint16) [n, k / group_size]: the per-group
 *   biases   step s and offset b (asymmetric min/max quantization: b is the
 *            group minimum, s = (max - min) / (2^bits - 1)).
 *   x        fp16 bit patterns, [m, k].
 *   y        fp32, [m, n].
 *
 * Common rules
 * ------------
 *   * Supported: bits in {2, 3, 4, 5, 6, 8}; group_size in {32, 64, 128}; k a positive
 *     multiple of 64 and of group_size; n, m >= 1 (m = 0 / t = 0 is accepted and does nothing).
 *   * Every tensor pointer is a DEVICE pointer owned by the caller and must
 *     stay valid until the stream reaches the launch.  Weights, activations,
 *     plans and workspaces must be 16-byte aligned; scales and biases 2-byte
 *     aligned (8-byte aligned arrays let the GEMM kernels load the scales of
 *     four groups at once; others take a slower per-group path); outputs
 *     4-byte (fp32) or 2-byte (fp16) aligned.
 *     Output buffers must not overlap inputs.
 *   * `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue
 *     work and return; results are valid once the stream is synchronized.
 *   * No entry point allocates device memory, frees it or synchronizes.
 *     Scratch memory comes from a caller-provided workspace whose size the
 *     matching *_workspace_size query returns.
 *   * Arguments are validated on the host before any HIP call, so every
 *     error status below can be produced without a GPU.  On error nothing is
 *     launched and qmm_last_error() describes the problem.
 *   * Thread safety: stateless apart from a thread-local error message;
 *     calls from several threads on several streams are safe.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QMM_OK = 0,
  QMM_ERR_INVALID_ARG = 1,  /* null / misaligned pointer, bad size, k % group_size != 0 */
  QMM_ERR_UNSUPPORTED = 2,  /* bits or group_size outside the supported set */
  QMM_ERR_WORKSPACE = 3,    /* workspace or plan buffer too small */
  QMM_ERR_HIP = 4           /* a HIP launch failed; text in qmm_last_error() */
} qmm_status;

/* hipStream_t, passed as an opaque pointer so that this header needs no HIP headers. */
typedef void* qmm_stream;

/* Library version, major * 10000 + minor * 100 + patch. */
int qmm_version(void);

/* Text of the last error raised on the calling thread ("" if none).  The
 * buffer is thread-local and static (BaseRT §3.2); it stays valid until the
 * next qmm_* call on the same thread. */
const char* qmm_last_error(void);

/* ------------------------------------------------------------ decode GEMV
 * y[n] = sum_k x[k] * W_hat[n, k]   (BaseRT §3.3: the M = 1 decode kernel)
 *   w       [n, k*bits/32] uint32 packed codes
 *   scales  [n, k/group_size] fp16 bits;  biases likewise
 *   x       [k] fp16 bits;  y [n] fp32 (overwritten)
 * Streams every weight byte once with 128-bit loads, unpacks and scales in
 * registers, reduces across lanes; small n gets an in-workgroup split of k.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int qmm_qgemv(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
              const uint16_t* x, float* y, int n, int k, int bits, int group_size,
              qmm_stream stream);

/* ---------------------------------------------------- batched decode GEMV
 * Many independent GEMVs (e.g. every projection of a decode step) in ONE
 * launch, which amortizes launch cost the way BaseRT §3 amortizes command
 * dispatch.  Two steps:
 *   1. qmm_qgemv_batched_plan (host only, no HIP call): from `count` problem
 *      descriptors (device pointers inside, host array) build a plan image
 *      in host memory `plan` of `plan_bytes`.  *plan_bytes_needed receives
 *      the size required; if plan is NULL or too small the call returns
 *      QMM_ERR_WORKSPACE without writing the plan.  All problems share bits
 *      and group_size; each has its own n and k.
 *   2. Copy the image verbatim to device memory (any copy), then call
 *      qmm_qgemv_batched with the device copy and the host image (whose
 *      64-byte header carries the launch geometry).  The plan stays valid
 *      while the pointers it names do; it can be launched any number of
 *      times.
 * Problems must not write overlapping y ranges.  Errors: INVALID_ARG,
 * UNSUPPORTED, WORKSPACE, HIP. */
typedef struct {
  const uint32_t* w;
  const uint16_t* scales;
  const uint16_t* biases;
  const uint16_t* x;
  float* y;
  int32_t n;
  int32_t k;
} qmm_gemv_problem;

int qmm_qgemv_batched_plan(const qmm_gemv_problem* problems, int count, int bits,
                           int group_size, void* plan, size_t plan_bytes,
                           size_t* plan_bytes_needed);
int qmm_qgemv_batched(const void* plan_device, const void* plan_host, qmm_stream stream);

/* ----------------------------------------------------------- prefill GEMM
 * y[m, n] = sum_k x[m, k] * W_hat[n, k]   (BaseRT §3.4: tiled prefill GEMM)
 *   x [m, k] fp16 bits; y [m, n] fp32 (overwritten); other operands as GEMV.
 * Weight tiles are dequantized to fp16 in registers (one rounding of
 * s*q + b) and multiplied on the fp16 matrix cores with fp32 accumulation.
 * workspace may be NULL when qmm_qgemm_workspace_size returns 0.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
size_t qmm_qgemm_workspace_size(int m, int n, int k, int bits, int group_size);
int qmm_qgemm(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
              const uint16_t* x, float* y, int m, int n, int k, int bits, int group_size,
              void* workspace, size_t workspace_bytes, qmm_stream stream);

/* ---------------------------------------------------- batched prefill GEMM
 * Several independent y_p = x_p W_hat_p^T (same arithmetic as qmm_qgemm) in
 * ONE launch: e.g. the q, k and v projections of a layer, or gate and up,
 * whose tiles together fill the chip where each alone would not (BaseRT
 * §3.4 tiled prefill GEMM; §3 amortized dispatch).  Two steps, as for the
 * batched GEMV:
 *   1. qmm_qgemm_batched_plan (host only, no HIP call): from `count`
 *      problem descriptors (device pointers, host array) choose one tile
 *      shape and k-split count for the batch and write the plan image into
 *      host memory `plan` of `plan_bytes`.  *plan_bytes_needed receives the
 *      image size and *workspace_bytes_needed the device workspace size
 *      (0 when k is not split); if plan is NULL or too small the call
 *      returns QMM_ERR_WORKSPACE without writing the image.  Each problem
 *      has its own m >= 0, n >= 1 and k (a multiple of 64); all share bits
 *      and group_size.  A problem with m = 0 is skipped (its x and y may be
 *      NULL).
 *   2. Copy the image verbatim to device memory (16-byte aligned), then
 *      call qmm_qgemm_batched with the device copy, the host image and the
 *      workspace.
 * Workspace (contents on entry do not matter): with k split, each split
 * writes an fp32 partial tile there and a second, short kernel adds the
 * partials of every tile in split order, so results are identical from run
 * to run.  Calls that share a workspace must not run concurrently.
 * Problems must not write overlapping y ranges.
 * Weight layout: `bits` alone means every w is row-major [n, k*bits/32] as
 * everywhere else; `bits | QMM_WEIGHTS_TILED` means every w was produced by
 * qmm_repack_tiled (then every n must be a multiple of 32), which the
 * prefill tiles read with fewer, fully contiguous loads.  Scales and biases
 * are row-major unless `bits` also carries QMM_SCALES_TILED: then every
 * `scales` pointer is an interleaved scale-and-bias array produced by
 * qmm_repack_scales_tiled (16-byte aligned; `biases` is not read and may be
 * NULL), which needs QMM_WEIGHTS_TILED, group_size 64, 2- to 8-bit codes and
 * k a multiple of 256.  The two scale layouts give identical results.  The
 * flag is taken the same way by qmm_qgemm and by the grouped MoE calls
 * (qmm_qgemm_grouped, _noalloc, _routed and qmm_moe_gate_up_swiglu, whose
 * stacked expert scales [E, n, k/64] repack as one [E*n, k/64] array).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
#define QMM_WEIGHTS_TILED 0x100
#define QMM_SCALES_TILED 0x200
typedef struct {
  const uint32_t* w;
  const uint16_t* scales;
  const uint16_t* biases;
  const uint16_t* x;
  float* y;
  int32_t m;
  int32_t n;
  int32_t k;
} qmm_gemm_problem;

int qmm_qgemm_batched_plan(const qmm_gemm_problem* problems, int count, int bits,
                           int group_size, void* plan, size_t plan_bytes,
                           size_t* plan_bytes_needed, size_t* workspace_bytes_needed);
int qmm_qgemm_batched(const void* plan_device, const void* plan_host, void* workspace,
                      size_t workspace_bytes, qmm_stream stream);

/* --------------------------------------------- mixture-of-experts grouped
 * BaseRT (native-Metal LLM inference on Apple Silicon), abstract and Fig. 1:
 * the mixture-of-experts prefill (Qwen3-30B-A3B, 4-bit) is where the pages
 * report their larger advantage; they give no mechanism, so the one here is
 * token-to-expert bucketing with one tile schedule per expert.  §3.3 applies
 * as for the GEMM (dequantization inside the inner loop).
 *
 * Pair p = t * top_k + j routes token t to expert e = expert_ids[t, j]:
 *     y[p, n] = sum_k A[row(p), k] * W_hat_e[n, k]
 *   w       [E, n, k*bits/32]; scales, biases [E, n, k/group_size]
 *   a       fp16 bits; a_row_per_pair = 0: A is [T, k] and row(p) = p / top_k
 *           (gate / up projections read the token); 1: A is [T*top_k, k] and
 *           row(p) = p (the down projection reads the pair's own row)
 *   expert_ids [T, top_k] int32, each in [0, E).  A pair whose id lies outside
 *           that range is not computed: its output row is NaN, and the count
 *           of such pairs is recorded in the plan header (below).
 *   y       [T*top_k, n] fp32 (overwritten)
 * Device-side token-to-expert bucketing (histogram, scan, scatter) builds
 * one tile list per expert in the workspace; the grouped GEMM then gathers
 * A rows, dequantizes that expert's weight tiles and scatters output rows.
 * The workspace size depends only on (T, top_k, E); n, k, bits and
 * group_size are accepted so that a caller can size it from the same
 * arguments as the product.
 *
 * Routing plan / workspace image (device memory, int32 words):
 *   word 0  row tiles in the list     word 1  rows per row tile
 *   word 2  pairs (T * top_k)         word 3  experts E
 *   word 4  pairs whose expert id was outside [0, E)  (byte offset 16)
 *   words 5..7 zero; then the bucketed pair list, the row-tile list and
 *   the per-chunk expert counts that the bucketing launches pass between them.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
size_t qmm_qgemm_grouped_workspace_size(int t, int top_k, int e, int n, int k, int bits,
                                        int group_size);
int qmm_qgemm_grouped(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                      const uint16_t* a, int a_row_per_pair, const int32_t* expert_ids,
                      float* y, int t, int top_k, int e, int n, int k, int bits,
                      int group_size, void* workspace, size_t workspace_bytes,
                      qmm_stream stream);

/* Allocation-free grouped product, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): qmm_qgemm_grouped with the same arguments minus the
 * workspace.  Its bucket lists and tile list live in a static device array
 * of QMM_GROUPED_SCRATCH_BYTES (1 MiB) that each GPU holds from the first
 * call on it until the process ends; the call allocates nothing, frees
 * nothing and calls no allocating library routine.  The scratch serves
 * every (t, top_k, e) whose qmm_qgemm_grouped_workspace_size is at most
 * 1 MiB (up to about 231,000 pairs, e.g. 28,900 tokens at top-8, with
 * E = 128); larger problems are refused with QMM_ERR_WORKSPACE before any
 * launch.  Every call on one GPU shares that GPU's array, so calls that
 * overlap on one GPU (several streams, several host threads) race and must
 * be serialized by the caller; the array is never cleared (each call
 * rewrites every word it reads).  Pairs with an out-of-range expert id get
 * NaN rows as in qmm_qgemm_grouped; their count stays in the scratch and is
 * not reported.  Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
#define QMM_GROUPED_SCRATCH_BYTES (1u << 20)
int qmm_qgemm_grouped_noalloc(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                              const uint16_t* a, int a_row_per_pair, const int32_t* expert_ids,
                              float* y, int t, int top_k, int e, int n, int k, int bits,
                              int group_size, qmm_stream stream);

/* Routing plan shared by the grouped products of one MoE layer (BaseRT,
 * abstract and Fig. 1: MoE prefill; §3 amortized dispatch).  Gate, up and
 * down read the same expert ids, so the token-to-expert bucketing (the first
 * launch of qmm_qgemm_grouped) can run once:
 *   qmm_moe_route        buckets expert_ids [T, top_k] into `plan` (device
 *                        memory of qmm_moe_route_size(T, top_k, E) bytes,
 *                        16-byte aligned, caller-owned; contents on entry
 *                        do not matter);
 *   qmm_qgemm_grouped_routed  the grouped product of qmm_qgemm_grouped, with
 *                        the same arguments except that `plan` and its size
 *                        `plan_bytes` replace expert_ids and the workspace.
 * The plan stays valid while expert_ids is unchanged, for any n, k, bits and
 * group size, and may be read by several launches in flight.  plan_bytes
 * below qmm_moe_route_size(T, top_k, E) is refused on the host (WORKSPACE);
 * a plan built for another (T, top_k, E) or another row tile is detected on
 * the device and the whole output is then written as NaN.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
size_t qmm_moe_route_size(int t, int top_k, int e);
int qmm_moe_route(const int32_t* expert_ids, int t, int top_k, int e, void* plan,
                  size_t plan_bytes, qmm_stream stream);
int qmm_qgemm_grouped_routed(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                             const uint16_t* a, int a_row_per_pair, const void* plan,
                             size_t plan_bytes, float* y, int t, int top_k, int e, int n, int k,
                             int bits, int group_size, qmm_stream stream);

/* Mixture-of-experts FFN block around the grouped products (BaseRT §3.3:
 * the FFN's matmuls and activation fused into fewer kernels; abstract and
 * Fig. 1: MoE prefill).
 *   qmm_moe_gate_up_swiglu  for every pair p (token row p / top_k of x
 *       [T, k] fp16), with e = the pair's expert from `plan` (qmm_moe_route,
 *       plan_bytes as for qmm_qgemm_grouped_routed):
 *           h[p, c] = fp16( silu(g) * u ),  silu(g) = g / (1 + exp(-g)),
 *           g = sum_k x[row, k] W_gate_e[c, k],  u = likewise with W_up_e
 *       (g, u and the SwiGLU in fp32; one rounding to fp16).  w_gate, w_up
 *       [E, n, k*bits/32] with their scales and biases as in
 *       qmm_qgemm_grouped; h [T*top_k, n] fp16 bits (overwritten) is the
 *       down projection's A (a_row_per_pair = 1).  bits = 16: fp16 weights.
 *       Rows of pairs with an out-of-range expert id, and all of h when the
 *       plan was built for other counts, are written as fp16 NaN.
 *   qmm_moe_combine  y[t, c] = sum_{j < top_k} weights[t, j] * y_pairs[t*top_k + j, c]
 *       with the slots added in order j = 0, 1, ... (fp32 fma), so the result
 *       does not depend on scheduling.  y_pairs [T*top_k, n] fp32 (the down
 *       projection's output), weights [T, top_k] fp32, y [T, n] fp32.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE (plan too small), HIP. */
int qmm_moe_gate_up_swiglu(const uint32_t* w_gate, const uint16_t* s_gate, const uint16_t* b_gate,
                           const uint32_t* w_up, const uint16_t* s_up, const uint16_t* b_up,
                           const uint16_t* x, const void* plan, size_t plan_bytes, uint16_t* h,
                           int t, int top_k, int e, int n, int k, int bits, int group_size,
                           qmm_stream stream);
int qmm_moe_combine(const float* y_pairs, const float* weights, float* y, int t, int top_k, int n,
                    qmm_stream stream);

/* ------------------------------------------------ load-time quantization
 * Asymmetric min/max quantization of a dense fp32 weight W[n, k] into the
 * packed format above: per group, s = fp16((max - min) / L) and
 * b = fp16(min) with L = 2^bits - 1 (fp32 arithmetic, IEEE division,
 * round-to-nearest-even), q = clamp(rint((w - b) / s), 0, L), and q = 0 for
 * every element when s == 0.  Work done once when a model is loaded
 * (BaseRT §3.2 prepares everything at load time).
 *   w_f32 [n, k] fp32; words [n, k*bits/32]; scales, biases [n, k/gs] fp16 bits.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int qmm_quantize(const float* w_f32, uint32_t* words, uint16_t* scales, uint16_t* biases,
                 int n, int k, int bits, int group_size, qmm_stream stream);

/* bf16 weights (load time).  The matrix cores multiply fp16 by fp16 or bf16
 * by bf16, not fp16 activations by bf16 weights, so bf16 weights are
 * converted once to fp16 and then used as bits = 16:
 *   dst[i] = fp16(bf16 src[i]), round to nearest even; exact for every bf16
 *   whose magnitude lies in fp16's normal range, +-inf beyond 65504.
 *   src, dst: count uint16 bit patterns (count even, 4-byte aligned; dst may
 *   equal src for an in-place conversion).
 * Errors: INVALID_ARG, HIP. */
int qmm_convert_bf16(const uint16_t* src, uint16_t* dst, size_t count, qmm_stream stream);

/* Tile-interleaved weights for the batched prefill GEMM (load time; a
 * layout of this library's own, not from the pages): out holds the same
 * words as the row-major w [n, k*bits/32], each 64-code group moved whole:
 *   group g of column c: w word (c * G + g) * WPG
 *                     -> out word ((c / 32) * G * 32 + g * 32 + c % 32) * WPG
 *   with G = k / 64 and WPG = 2 * bits words per group (32 for bits = 16),
 * so the 32 columns of one matrix-core column block are contiguous for each
 * group.  n must be a multiple of 32 and k of 64; w and out are device
 * buffers of n * k * bits / 8 bytes (16-byte aligned, not overlapping); out
 * is used with QMM_WEIGHTS_TILED: on the bits of qmm_qgemm, of a batched
 * plan, of qmm_qgemm_grouped, qmm_qgemm_grouped_routed and
 * qmm_moe_gate_up_swiglu (stacked experts [E, n, ...] repack as one
 * [E*n, ...] matrix, which keeps each expert's block whole when n is a
 * multiple of 32).  The decode GEMV keeps reading row-major weights.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int qmm_repack_tiled(const uint32_t* w, uint32_t* out, int n, int k, int bits, qmm_stream stream);

/* Interleaved scales and biases for the prefill GEMM over tile-interleaved
 * weights (load time; a layout of this library's own, not from the pages):
 * out holds every scale and bias of the row-major scales and biases
 * [n, k/64] (groups of 64 codes), for each block of 32 columns and each
 * quad of 4 groups the 32 columns' 16-byte {s[4q .. 4q+3], b[4q .. 4q+3]}
 * next to each other:
 *   scales[c * G + g] -> out[((c / 32) * (G / 4) * 32 + c % 32) * 8 + (g / 4) * 256 + g % 4]
 *   biases[c * G + g] -> the same index + 4,      with G = k / 64,
 * so one wave's scale loads read whole lines.  n must be a multiple of 32 and
 * k of 256; scales and biases are device arrays of n * k / 64 fp16 (2-byte
 * aligned), out one of 2 * n * k / 64 fp16 (16-byte aligned, overlapping
 * neither); out is used as `scales` with QMM_SCALES_TILED (stacked MoE expert
 * scales and biases [E, n, k/64] repack as one [E*n, k/64] matrix, which
 * keeps each expert's block whole when n is a multiple of 32).
 * Errors: INVALID_ARG, HIP. */
int qmm_repack_scales_tiled(const uint16_t* scales, const uint16_t* biases, uint16_t* out, int n, int k,
                            qmm_stream stream);

/* ------------------------------------------------------------- diagnostics
 * Expose the device-side stages of the hot path for bit-exact checking.
 * qmm_unpack_codes: codes[n, k] (uint8) = the codes of `w`, decoded with
 *   the same register unpack the GEMV and GEMM kernels use.
 * qmm_dequant: out[n, k] = W_hat as fp32 (out_is_f16 = 0; one rounding of
 *   the exact s*q + b) or as fp16 bits (out_is_f16 = 1; one rounding, the
 *   value the GEMM feeds to the matrix cores).
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int qmm_unpack_codes(const uint32_t* w, uint8_t* codes, int n, int k, int bits,
                     qmm_stream stream);
int qmm_dequant(const uint32_t* w, const uint16_t* scales, const uint16_t* biases,
                void* out, int out_is_f16, int n, int k, int bits, int group_size,
                qmm_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
