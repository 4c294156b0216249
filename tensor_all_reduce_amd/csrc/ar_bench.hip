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

// Flat copy, one 16-byte group per lane, non-temporal loads and stores: the
// fastest plain copy measured on MI355X (the attainable-bandwidth reference).
__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                              size_t nvec) {
  const size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v < nvec) __builtin_nontemporal_store(__builtin_nontemporal_load(src + v), dst + v);
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
  (void)hipEventRecord(e0, s);
  for (int i = 0; i < iters; ++i) {
    int rc = call(which, ins, outs, P, n, scratch, stream);
    if (rc) return rc;
  }
  (void)hipEventRecord(e1, s);
  (void)hipEventSynchronize(e1);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
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
  (void)hipStreamSynchronize(s);
  for (int i = 0; i < iters; ++i) {
    auto a = std::chrono::steady_clock::now();
    int rc = call(which, ins, outs, P, n, scratch, stream);
    if (rc) return rc;
    (void)hipStreamSynchronize(s);
    auto b = std::chrono::steady_clock::now();
    t[i] = std::chrono::duration<double, std::micro>(b - a).count();
  }
  std::sort(t.begin(), t.end());
  *p50 = t[t.size() / 2];
  *p10 = t[t.size() / 10];
  *p90 = t[(t.size() * 9) / 10];
  return AR_OK;
}

// Plain device copy of `bytes` (a multiple of 16, 16-byte aligned buffers),
// `block` lanes per workgroup (64, 128 or 256).
int arb_copy(const void* src, void* dst, size_t bytes, int block, void* stream) {
  if ((bytes & 15u) || !src || !dst || (block != 64 && block != 128 && block != 256))
    return AR_ERR_INVALID;
  const size_t nvec = bytes / 16;
  const size_t grid = (nvec + block - 1) / block;
  if (grid == 0 || grid > 0x7FFFFFFFull) return AR_ERR_INVALID;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)grid), dim3(block), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

}  // extern "C"
