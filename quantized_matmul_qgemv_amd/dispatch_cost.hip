// Host cost of one call of each C ABI entry point, measured without Python.
//
// BaseRT (native-Metal LLM inference on Apple Silicon) §3 puts the CPU-side
// dispatch on the decode hot path: every decode step issues its kernels from
// the host, so the cost of argument checks, geometry choice and the launch
// itself is paid per token.  This program times, for each entry point, a
// loop of back-to-back calls on one stream (host wall time of the loop
// divided by the calls; the GPU work of each call is a few microseconds so
// the launch queue never fills) and, as the floor, the same loop launching
// an empty kernel with hipLaunchKernelGGL.  Operands are zero-filled device
// buffers of small shapes (valid inputs: zero codes, scales and biases).
// Output: one JSON object on stdout, microseconds per call (median of 7
// repetitions of 200 calls).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <chrono>
#include <functional>
#include <string>
#include <vector>

#include "qmm.h"

namespace {

__global__ void empty_kernel(float* p) {
  if (p != nullptr && threadIdx.x == 1023) p[0] = 0.0f;  // never taken (64 threads)
}

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    exit(2);
  }
}

void qmm_ok(int st, const char* what) {
  if (st != QMM_OK) {
    fprintf(stderr, "%s: status %d: %s\n", what, st, qmm_last_error());
    exit(3);
  }
}

void* dalloc(size_t bytes) {
  void* p = nullptr;
  hip_check(hipMalloc(&p, bytes), "hipMalloc");
  hip_check(hipMemset(p, 0, bytes), "hipMemset");
  return p;
}

double us_per_call(hipStream_t st, const std::function<void()>& call) {
  constexpr int kCalls = 200, kReps = 7;
  for (int i = 0; i < 20; ++i) call();  // warm-up (first-call set-up, caches)
  hip_check(hipStreamSynchronize(st), "sync");
  std::vector<double> us;
  for (int r = 0; r < kReps; ++r) {
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < kCalls; ++i) call();
    const auto t1 = std::chrono::steady_clock::now();
    hip_check(hipStreamSynchronize(st), "sync");
    us.push_back(std::chrono::duration<double, std::micro>(t1 - t0).count() / kCalls);
  }
  std::sort(us.begin(), us.end());
  return us[kReps / 2];
}

}  // namespace

int main() {
  hipStream_t st;
  hip_check(hipStreamCreate(&st), "hipStreamCreate");
  const qmm_stream qs = (qmm_stream)st;

  // GEMV 1024 x 1024, 4-bit, groups of 64
  const int n = 1024, k = 1024;
  uint32_t* w = (uint32_t*)dalloc((size_t)n * k / 2);
  uint16_t* s = (uint16_t*)dalloc((size_t)n * (k / 64) * 2);
  uint16_t* b = (uint16_t*)dalloc((size_t)n * (k / 64) * 2);
  uint16_t* x = (uint16_t*)dalloc((size_t)64 * k * 2);
  float* y = (float*)dalloc((size_t)64 * n * 4 * 3);

  // batched GEMV plan: 7 problems over the same operands (distinct outputs)
  qmm_gemv_problem vp[7];
  for (int i = 0; i < 7; ++i) vp[i] = qmm_gemv_problem{w, s, b, x, y + (size_t)i * n, n, k};
  size_t vneed = 0;
  qmm_qgemv_batched_plan(vp, 7, 4, 64, nullptr, 0, &vneed);
  std::vector<unsigned char> vplan_host(vneed);
  qmm_ok(qmm_qgemv_batched_plan(vp, 7, 4, 64, vplan_host.data(), vneed, &vneed), "gemv plan");
  void* vplan_dev = dalloc(vneed);
  hip_check(hipMemcpy(vplan_dev, vplan_host.data(), vneed, hipMemcpyHostToDevice), "copy plan");

  // GEMM 64 x 1024 x 1024 and a batched plan of three such problems
  const int m = 64;
  const size_t gws = qmm_qgemm_workspace_size(m, n, k, 4, 64);
  void* gwsp = gws ? dalloc(gws) : nullptr;
  qmm_gemm_problem gp[3];
  for (int i = 0; i < 3; ++i) gp[i] = qmm_gemm_problem{w, s, b, x, y + (size_t)i * m * n, m, n, k};
  size_t gneed = 0, gwneed = 0;
  qmm_qgemm_batched_plan(gp, 3, 4, 64, nullptr, 0, &gneed, &gwneed);
  std::vector<unsigned char> gplan_host(gneed);
  qmm_ok(qmm_qgemm_batched_plan(gp, 3, 4, 64, gplan_host.data(), gneed, &gneed, &gwneed), "gemm plan");
  void* gplan_dev = dalloc(gneed);
  hip_check(hipMemcpy(gplan_dev, gplan_host.data(), gneed, hipMemcpyHostToDevice), "copy plan");
  void* gbws = dalloc(gwneed > 16 ? gwneed : 16);

  // MoE: 16 tokens, top-2 of 8 experts, 256 x 256 expert weights
  const int t = 16, top_k = 2, e = 8, en = 256, ek = 256;
  uint32_t* ew = (uint32_t*)dalloc((size_t)e * en * ek / 2);
  uint16_t* es = (uint16_t*)dalloc((size_t)e * en * (ek / 64) * 2);
  int32_t* ids = (int32_t*)dalloc((size_t)t * top_k * 4);
  float* ey = (float*)dalloc((size_t)t * top_k * en * 4);
  const size_t rsz = qmm_moe_route_size(t, top_k, e);
  void* plan = dalloc(rsz);
  void* mws = dalloc(qmm_qgemm_grouped_workspace_size(t, top_k, e, en, ek, 4, 64));
  const size_t mwsz = qmm_qgemm_grouped_workspace_size(t, top_k, e, en, ek, 4, 64);
  qmm_ok(qmm_moe_route(ids, t, top_k, e, plan, rsz, qs), "route");

  const double floor_us = us_per_call(st, [&] {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, st, y);
  });
  const double gemv_us = us_per_call(st, [&] { qmm_ok(qmm_qgemv(w, s, b, x, y, n, k, 4, 64, qs), "qgemv"); });
  const double gemv_b_us = us_per_call(st, [&] {
    qmm_ok(qmm_qgemv_batched(vplan_dev, vplan_host.data(), qs), "qgemv_batched");
  });
  const double gemm_us = us_per_call(st, [&] {
    qmm_ok(qmm_qgemm(w, s, b, x, y, m, n, k, 4, 64, gwsp, gws, qs), "qgemm");
  });
  const double gemm_b_us = us_per_call(st, [&] {
    qmm_ok(qmm_qgemm_batched(gplan_dev, gplan_host.data(), gbws, gwneed > 16 ? gwneed : 16, qs),
           "qgemm_batched");
  });
  const double route_us = us_per_call(st, [&] { qmm_ok(qmm_moe_route(ids, t, top_k, e, plan, rsz, qs), "route"); });
  const double routed_us = us_per_call(st, [&] {
    qmm_ok(qmm_qgemm_grouped_routed(ew, es, es, x, 0, plan, rsz, ey, t, top_k, e, en, ek, 4, 64, qs),
           "grouped_routed");
  });
  const double grouped_us = us_per_call(st, [&] {
    qmm_ok(qmm_qgemm_grouped(ew, es, es, x, 0, ids, ey, t, top_k, e, en, ek, 4, 64, mws, mwsz, qs),
           "grouped");
  });
  // host-only steps: plan building (no HIP call)
  auto host_only = [](const std::function<void()>& f) {
    for (int i = 0; i < 20; ++i) f();
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < 1000; ++i) f();
    const auto t1 = std::chrono::steady_clock::now();
    return std::chrono::duration<double, std::micro>(t1 - t0).count() / 1000;
  };
  const double vplan_us = host_only([&] {
    qmm_ok(qmm_qgemv_batched_plan(vp, 7, 4, 64, vplan_host.data(), vneed, &vneed), "gemv plan");
  });
  const double gplan_us = host_only([&] {
    qmm_ok(qmm_qgemm_batched_plan(gp, 3, 4, 64, gplan_host.data(), gneed, &gneed, &gwneed), "gemm plan");
  });
  hip_check(hipStreamSynchronize(st), "sync");
  printf("{\"unit\": \"us host time per call\", \"calls\": 200, \"reps\": 7, "
         "\"empty_kernel_launch\": %.3f, \"qmm_qgemv\": %.3f, \"qmm_qgemv_batched\": %.3f, "
         "\"qmm_qgemm\": %.3f, \"qmm_qgemm_batched\": %.3f, \"qmm_moe_route\": %.3f, "
         "\"qmm_qgemm_grouped_routed\": %.3f, \"qmm_qgemm_grouped\": %.3f, "
         "\"qmm_qgemv_batched_plan_7\": %.3f, \"qmm_qgemm_batched_plan_3\": %.3f}\n",
         floor_us, gemv_us, gemv_b_us, gemm_us, gemm_b_us, route_us, routed_us, grouped_us, vplan_us,
         gplan_us);
  return 0;
}
