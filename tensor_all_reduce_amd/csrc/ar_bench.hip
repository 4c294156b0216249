// Measurement helpers for the bench (libarbench.so): native timing loops
// around the C-ABI entry points, so per-call latency excludes Python, and a
// plain copy kernel of known size that calibrates the memory counters and
// measures the attainable HBM bandwidth.  Not part of the reduction library.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <vector>

#include "ar.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                              size_t nvec) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) dst[v] = src[v];
}

int call(int which, const void* const* ins, void* const* outs, int P, size_t n, void* scratch,
         void* stream) {
  switch (which) {
    case 0: return ar_reduce_oneshot(ins, P, outs[0], n, stream);
    case 1: return ar_reduce_2stage(ins, outs, P, n, nullptr, stream);
    case 2: return ar_reduce_2stage(ins, outs, P, n, scratch, stream);
    default: return AR_ERR_INVALID;
  }
}

}  // namespace

extern "C" {

// Average stream time per call, in microseconds, of `iters` back-to-back
// calls (launch included), bracketed by HIP events on `stream`.
// which: 0 one-shot (outs[0]), 1 two-stage fused, 2 two-stage staged.
// Returns a negative status on error.
double arb_stream_us(int which, const void* const* ins, void* const* outs, int P, size_t n,
                     void* scratch, int iters, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return AR_ERR_HIP;
  for (int i = 0; i < 20; ++i) {
    int rc = call(which, ins, outs, P, n, scratch, stream);
    if (rc) return rc;
  }
  hipEventRecord(e0, s);
  for (int i = 0; i < iters; ++i) {
    int rc = call(which, ins, outs, P, n, scratch, stream);
    if (rc) return rc;
  }
  hipEventRecord(e1, s);
  hipEventSynchronize(e1);
  float ms = 0.f;
  hipEventElapsedTime(&ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return 1000.0 * (double)ms / iters;
}

// Single-call wall latency: C-ABI call -> hipStreamSynchronize return,
// host steady clock; writes the median, 10th and 90th percentiles (us).
int arb_wall_us(int which, const void* const* ins, void* const* outs, int P, size_t n, void* scratch,
                int iters, void* stream, double* p50, double* p10, double* p90) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<double> t(iters > 0 ? iters : 1);
  for (int i = 0; i < 20; ++i) {
    int rc = call(which, ins, outs, P, n, scratch, stream);
    if (rc) return rc;
  }
  hipStreamSynchronize(s);
  for (int i = 0; i < iters; ++i) {
    auto a = std::chrono::steady_clock::now();
    int rc = call(which, ins, outs, P, n, scratch, stream);
    if (rc) return rc;
    hipStreamSynchronize(s);
    auto b = std::chrono::steady_clock::now();
    t[i] = std::chrono::duration<double, std::micro>(b - a).count();
  }
  std::sort(t.begin(), t.end());
  *p50 = t[t.size() / 2];
  *p10 = t[t.size() / 10];
  *p90 = t[(t.size() * 9) / 10];
  return AR_OK;
}

// Plain device copy of `bytes` (a multiple of 16, 16-byte aligned buffers).
int arb_copy(const void* src, void* dst, size_t bytes, int grid, void* stream) {
  if ((bytes & 15u) || !src || !dst) return AR_ERR_INVALID;
  hipLaunchKernelGGL(k_copy, dim3(grid > 0 ? grid : 1024), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

}  // extern "C"
