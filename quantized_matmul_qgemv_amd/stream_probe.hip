// Plain streaming rates of the GPU this runs on, as a scale for the decode
// GEMV's bandwidth: how fast a kernel that only reads memory (16-byte loads,
// no arithmetic beyond an XOR that keeps the loads alive) streams a given
// number of bytes, and how fast a plain copy runs.  Not part of the library:
// a measurement harness that bench.py runs beside the decode figure.
//
// usage: qmm_stream_probe BYTES
// Two buffers of BYTES each (together larger than the 256 MB last-level
// cache for the decode pass's 338 MB) alternate between launches, so every
// launch reads from HBM.  Each grid shape (workgroups x 256 threads, 4
// independent 16-byte loads per thread per loop trip, consecutive lanes
// reading consecutive 16-byte pieces) is timed over 20 launches between two
// HIP events after 3 warm-up launches, once with ordinary loads and once
// with non-temporal ones (the nt cache policy: lines not kept for reuse).
// Output: one JSON object on stdout with GB/s per grid and policy and the
// best of each policy.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <string>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void read_stream(const u32x4* __restrict__ p, size_t n16,
                                                   unsigned* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v = load16<NT>(p + i) ^ load16<NT>(p + i + stride) ^ load16<NT>(p + i + 2 * stride) ^
                    load16<NT>(p + i + 3 * stride);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = load16<NT>(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // the buffers hold zeros, so this store never happens; the compiler
  // cannot know that and keeps every load
  if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    exit(2);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const size_t bytes = argc > 1 ? strtoull(argv[1], nullptr, 10) : (size_t)337800704;
  const size_t n16 = bytes / 16;
  if (n16 == 0) {
    fprintf(stderr, "BYTES must be at least 16\n");
    return 2;
  }
  u32x4* buf[2];
  unsigned* out;
  for (auto& b : buf) {
    check(hipMalloc(&b, n16 * 16), "hipMalloc");
    check(hipMemset(b, 0, n16 * 16), "hipMemset");
  }
  const int kMaxGrid = 256 * 64;
  check(hipMalloc(&out, kMaxGrid * sizeof(unsigned)), "hipMalloc");
  hipStream_t st;
  check(hipStreamCreate(&st), "hipStreamCreate");
  hipEvent_t e0, e1;
  check(hipEventCreate(&e0), "event");
  check(hipEventCreate(&e1), "event");

  std::string json = "{\"unit\": \"GB/s of bytes read\", \"bytes\": " + std::to_string(n16 * 16) +
                     ", \"threads_per_workgroup\": 256";
  const int grids[] = {256 * 2, 256 * 4, 256 * 8, 256 * 16, 256 * 32, 256 * 64};
  for (int nt = 0; nt < 2; ++nt) {
    void (*kern)(const u32x4*, size_t, unsigned*) = nt ? read_stream<true> : read_stream<false>;
    const char* tag = nt ? "_nt" : "";
    json += std::string(", \"by_workgroups") + tag + "\": {";
    double best = 0.0;
    int best_grid = 0;
    bool first = true;
    for (int grid : grids) {
      for (int i = 0; i < 3; ++i) hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, buf[i & 1], n16, out);
      check(hipStreamSynchronize(st), "warm-up");
      constexpr int kReps = 20;
      check(hipEventRecord(e0, st), "record");
      for (int i = 0; i < kReps; ++i) hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, buf[i & 1], n16, out);
      check(hipEventRecord(e1, st), "record");
      check(hipEventSynchronize(e1), "sync");
      check(hipGetLastError(), "launch");
      float ms = 0.0f;
      check(hipEventElapsedTime(&ms, e0, e1), "elapsed");
      const double gbs = (double)(n16 * 16) / (ms / kReps * 1e-3) / 1e9;
      if (gbs > best) {
        best = gbs;
        best_grid = grid;
      }
      char item[96];
      snprintf(item, sizeof item, "%s\"%d\": %.1f", first ? "" : ", ", grid, gbs);
      json += item;
      first = false;
    }
    char tail[160];
    snprintf(tail, sizeof tail, "}, \"best%s_gb_per_s\": %.1f, \"best%s_workgroups\": %d", tag, best, tag,
             best_grid);
    json += tail;
  }
  json += "}";
  printf("%s\n", json.c_str());
  return 0;
}
