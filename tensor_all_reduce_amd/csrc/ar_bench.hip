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

// N buffers copied side by side: out[j] = in[j] for j < N, the same access
// pattern as an N -> N reduce (N read streams and N write streams at the same
// offsets) with no arithmetic.  64-lane workgroups; each lane moves V groups
// of 16 bytes per buffer, strided by the workgroup so that each wavefront
// instruction covers one contiguous 1 KiB span.  The attainable bandwidth of
// the pattern, as the plain copy is that of a single stream.
struct MultiPtrs {
  const u32x4* in[8];
  u32x4* out[8];
};

template <int N, int V>
__global__ __launch_bounds__(64) void k_copy_multi(MultiPtrs m, size_t nvec) {
  const size_t b0 = (size_t)blockIdx.x * 64 * V + threadIdx.x;
  u32x4 a[V][N];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t v = b0 + (size_t)u * 64;
    if (v < nvec) {
#pragma unroll
      for (int j = 0; j < N; ++j) a[u][j] = __builtin_nontemporal_load(m.in[j] + v);
    }
  }
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t v = b0 + (size_t)u * 64;
    if (v < nvec) {
#pragma unroll
      for (int j = 0; j < N; ++j) __builtin_nontemporal_store(a[u][j], m.out[j] + v);
    }
  }
}

// The one-shot's access pattern without its arithmetic: N buffers read
// (non-temporal loads), their XOR written to one output, with the one-shot's
// tiling (64-lane workgroups, 1 KiB of every buffer each).
template <int N, bool NTS>
__global__ __launch_bounds__(64) void k_gather_xor(MultiPtrs m, size_t nvec) {
  const size_t v = (size_t)blockIdx.x * 64 + threadIdx.x;
  if (v >= nvec) return;
  u32x4 a[N];
#pragma unroll
  for (int j = 0; j < N; ++j) a[j] = __builtin_nontemporal_load(m.in[j] + v);
  u32x4 r = a[0];
#pragma unroll
  for (int j = 1; j < N; ++j) r ^= a[j];
  if constexpr (NTS) __builtin_nontemporal_store(r, m.out[0] + v);
  else m.out[0][v] = r;
}

// Consumer of a flagged chunked reduce.  Persistent grid (no LDS request,
// at most two workgroups per CU, so the producer's workgroups always fit
// beside it: a waiting grid that filled every wave slot would keep them
// out): workgroup b walks tiles b, b+G, ... (G = grid) in chunk order; a
// tile is 4 groups of 16 bytes per lane (16 KiB), so each chunk is spread
// over many workgroups and its consumer work over the whole GPU.  Before a
// tile, wavefront 0 polls done[first + c] with relaxed device-scope loads,
// sleeping between polls, at most max_spins times, then performs one
// device-scope acquire fence (an L1 and L2 invalidate; polling with acquire
// loads would invalidate the XCD's L2 on every spin, evicting the
// producer's lines while it runs); a workgroup barrier passes the
// acquired view on to the other wavefronts, which share the CU's L1.  The
// tile is copied from src to dst; with WORK, each lane also runs `work`
// dependent FMA rounds on the words it loaded (a compute-bound consumer)
// and stores its total to sink[b * 256 + lane].  A tile whose flag never
// arrived counts one timeout and is still copied (so a premature read shows
// up as wrong data).
template <bool WORK>
__global__ __launch_bounds__(256) void k_consume(const uint32_t* done, uint32_t epoch, const u32x4* src,
                                                 u32x4* dst, size_t nvec, size_t chunk_vec,
                                                 uint32_t first, uint32_t max_spins, uint32_t* timeouts,
                                                 int work, float* sink) {
  constexpr int V = 4;
  const size_t tile = (size_t)V * blockDim.x;
  const size_t tiles_per_chunk = (chunk_vec + tile - 1) / tile;
  const size_t nchunks = (nvec + chunk_vec - 1) / chunk_vec;
  const size_t ntiles = nchunks * tiles_per_chunk;
  float total = 0.0f;
  for (size_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const size_t c = t / tiles_per_chunk, k = t % tiles_per_chunk;
    if (threadIdx.x < 64) {
      uint32_t f = __hip_atomic_load(done + first + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (uint32_t s = 0; f != epoch && s < max_spins; ++s) {
        __builtin_amdgcn_s_sleep(2);
        f = __hip_atomic_load(done + first + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (f != epoch && threadIdx.x == 0) atomicAdd(timeouts, 1u);
    }
    __syncthreads();
    const size_t c1 = (c + 1) * chunk_vec < nvec ? (c + 1) * chunk_vec : nvec;
    const size_t b0 = c * chunk_vec + k * tile + threadIdx.x;
    u32x4 x[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const size_t v = b0 + (size_t)u * blockDim.x;
      if (v < c1) x[u] = src[v];
    }
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const size_t v = b0 + (size_t)u * blockDim.x;
      if (v < c1) {
        __builtin_nontemporal_store(x[u], dst + v);
        if constexpr (WORK) {
          // four independent chains, seeded in [1, 2) from the data
          float a = __uint_as_float((x[u].x & 0x007FFFFFu) | 0x3F800000u);
          float b = __uint_as_float((x[u].y & 0x007FFFFFu) | 0x3F800000u);
          float e = __uint_as_float((x[u].z & 0x007FFFFFu) | 0x3F800000u);
          float d = __uint_as_float((x[u].w & 0x007FFFFFu) | 0x3F800000u);
          for (int i = 0; i < work; ++i) {
            a = __builtin_fmaf(a, 0.999f, 0.001f);
            b = __builtin_fmaf(b, 0.998f, 0.002f);
            e = __builtin_fmaf(e, 0.997f, 0.003f);
            d = __builtin_fmaf(d, 0.996f, 0.004f);
          }
          total += (a + b) + (e + d);
        }
      }
    }
  }
  if constexpr (WORK) sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = total;
}

// One wavefront that sleeps `rounds` times (about 64 * 127 clocks each): a
// bounded delay at the head of a stream, so that the host can queue work
// behind it before the GPU reaches that work.
__global__ void k_delay(int rounds) {
  for (int i = 0; i < rounds; ++i) __builtin_amdgcn_s_sleep(127);
}

// Empty kernels with 0, 8 or 192 bytes of arguments: the host cost of a
// launch itself, against which the library's per-call host cost is read.
struct Arg8 { uint64_t a; };
struct Arg192 { uint64_t a[24]; };
__global__ void k_noarg() {}
__global__ void k_arg8(Arg8) {}
__global__ void k_arg192(Arg192) {}

// Read-only sweep: every lane loads 16-byte groups (non-temporal) and folds
// them with xor; one word per workgroup is written so the loads stay live.
// Measures the attainable read bandwidth beside the copy's read+write rate.
__global__ __launch_bounds__(256) void k_readsum(const u32x4* __restrict__ src, size_t nvec,
                                                 uint32_t* __restrict__ out) {
  constexpr int V = 4;
  const size_t b0 = (size_t)blockIdx.x * blockDim.x * V + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t v = b0 + (size_t)u * blockDim.x;
    if (v < nvec) acc ^= __builtin_nontemporal_load(src + v);
  }
  uint32_t w = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int o = 32; o > 0; o >>= 1) w ^= __shfl_xor(w, o, 64);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// ALU-bound stand-in for the partner ubatch's compute: `iters` rounds of
// dependent fused multiply-adds on four accumulators per lane; one float out.
__global__ __launch_bounds__(256) void k_alu(float* out, int iters) {
  float a = threadIdx.x * 1e-3f, b = 1.0f, c = 0.5f, d = 0.25f;
  for (int i = 0; i < iters; ++i) {
    a = __builtin_fmaf(a, 0.999f, 0.001f);
    b = __builtin_fmaf(b, 0.998f, 0.002f);
    c = __builtin_fmaf(c, 0.997f, 0.003f);
    d = __builtin_fmaf(d, 0.996f, 0.004f);
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = a + b + c + d;
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

// Events released on every return path.
struct EventPair {
  hipEvent_t a = nullptr, b = nullptr;
  bool ok = false;
  EventPair() { ok = hipEventCreate(&a) == hipSuccess && hipEventCreate(&b) == hipSuccess; }
  ~EventPair() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
  }
  // average microseconds per iteration between a and b, once b has completed
  double us_between(int iters) {
    (void)hipEventSynchronize(b);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, a, b);
    return 1000.0 * (double)ms / iters;
  }
};

// One decode all-reduce on fused payloads: P packs, error-record reset,
// recursive doubling, P unpacks (chain != 0); or the recursive doubling
// alone (chain == 0).
int decode_once(const void* const* x, void* const* y, uint64_t* const* w_in, uint64_t* const* w_out, int P,
                size_t n, uint32_t seq0, uint64_t* mailbox, int flags, uint64_t* d_err, int chain,
                void* stream) {
  int L = 0;
  while ((1 << L) < P) ++L;
  if (chain) {
    for (int p = 0; p < P; ++p) {
      int rc = ar_pack_fused(x[p], w_in[p], n, seq0, stream);
      if (rc) return rc;
    }
    int rc = ar_err_init(d_err, stream);
    if (rc) return rc;
  }
  int rc = ar_rd_schedule(w_in, w_out, P, n, seq0, mailbox, flags, d_err, stream);
  if (rc || !chain) return rc;
  for (int p = 0; p < P; ++p) {
    rc = ar_unpack_fused(w_out[p], y[p], n, seq0 + (uint32_t)L, d_err, stream);
    if (rc) return rc;
  }
  return AR_OK;
}

}  // namespace

extern "C" {

// Average stream time per call, in microseconds, of `iters` back-to-back
// calls (launch included), bracketed by HIP events on `stream`.
// which: 0 one-shot (outs[0]), 1 two-stage fused, 2 two-stage staged.
// Returns a negative status on error.
double arb_stream_us(int which, const void* const* ins, void* const* outs, int P, size_t n,
                     void* scratch, int iters, void* stream) {
  if (iters < 1) return AR_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  EventPair ev;
  if (!ev.ok) return AR_ERR_HIP;
  for (int i = 0; i < 20; ++i) {
    int rc = call(which, ins, outs, P, n, scratch, stream);
    if (rc) return rc;
  }
  (void)hipEventRecord(ev.a, s);
  for (int i = 0; i < iters; ++i) {
    int rc = call(which, ins, outs, P, n, scratch, stream);
    if (rc) return rc;
  }
  (void)hipEventRecord(ev.b, s);
  return ev.us_between(iters);
}

// Host time per call of `iters` back-to-back calls, the enqueue only (steady
// clock around the loop, no synchronisation inside it; the stream is drained
// before and after).  which 0..2 as for arb_stream_us; which = -1, -2, -3:
// an empty kernel with no, 8 or 192 bytes of arguments.
double arb_enqueue_us(int which, const void* const* ins, void* const* outs, int P, size_t n, void* scratch,
                      int iters, void* stream) {
  if (iters < 1 || which < -3 || which > 2) return AR_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto one = [&]() -> int {
    if (which >= 0) return call(which, ins, outs, P, n, scratch, stream);
    if (which == -1) hipLaunchKernelGGL(k_noarg, dim3(1), dim3(64), 0, s);
    else if (which == -2) hipLaunchKernelGGL(k_arg8, dim3(1), dim3(64), 0, s, Arg8{0});
    else hipLaunchKernelGGL(k_arg192, dim3(1), dim3(64), 0, s, Arg192{});
    return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
  };
  for (int i = 0; i < 20; ++i) {
    int rc = one();
    if (rc) return rc;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return AR_ERR_HIP;
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < iters; ++i) {
    int rc = one();
    if (rc) return rc;
  }
  const auto t1 = std::chrono::steady_clock::now();
  if (hipStreamSynchronize(s) != hipSuccess) return AR_ERR_HIP;
  return std::chrono::duration<double, std::micro>(t1 - t0).count() / iters;
}

// Single-call wall latency: C-ABI call -> hipStreamSynchronize return,
// host steady clock; writes the median, 10th and 90th percentiles (us).
int arb_wall_us(int which, const void* const* ins, void* const* outs, int P, size_t n, void* scratch,
                int iters, void* stream, double* p50, double* p10, double* p90) {
  if (iters < 1 || !p50 || !p10 || !p90) return AR_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<double> t(iters);
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

// Like arb_stream_us, but call k works on the k % nsets-th of nsets
// disjoint element ranges: every buffer pointer is advanced by
// (k % nsets) * stride_elems bf16 elements.  With a footprint above the
// 256 MiB last-level cache this measures the cold (HBM) cost of small
// calls.  which: 0 one-shot (outs[0]), 1 two-stage fused.
double arb_stream_rot_us(int which, const void* const* ins, void* const* outs, int P, size_t n,
                         size_t stride_elems, int nsets, int iters, void* stream) {
  if (which < 0 || which > 1 || P < 1 || P > AR_MAX_RANKS || nsets < 1 || iters < 1 || stride_elems < n)
    return AR_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  EventPair ev;
  if (!ev.ok) return AR_ERR_HIP;
  const void* in_k[AR_MAX_RANKS];
  void* out_k[AR_MAX_RANKS];
  auto one = [&](int k) {
    const size_t off = (size_t)(k % nsets) * stride_elems * 2;
    for (int p = 0; p < P; ++p) {
      in_k[p] = static_cast<const char*>(ins[p]) + off;
      out_k[p] = static_cast<char*>(outs[p]) + off;
    }
    return call(which, in_k, out_k, P, n, nullptr, stream);
  };
  for (int i = 0; i < 2 * nsets; ++i) {
    int rc = one(i);
    if (rc) return rc;
  }
  (void)hipEventRecord(ev.a, s);
  for (int i = 0; i < iters; ++i) {
    int rc = one(i);
    if (rc) return rc;
  }
  (void)hipEventRecord(ev.b, s);
  return ev.us_between(iters);
}

// Average stream time, in microseconds, of `iters` back-to-back decode
// all-reduces on fused payloads (see decode_once; seq0 = 1 throughout, so
// d_err stays zero when every payload is valid).  mailbox NULL: fused
// recursive doubling; non-NULL: staged.
double arb_decode_us(const void* const* x, void* const* y, uint64_t* const* w_in, uint64_t* const* w_out,
                     int P, size_t n, uint64_t* mailbox, int flags, uint64_t* d_err, int chain, int iters,
                     void* stream) {
  if (iters < 1) return AR_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  EventPair ev;
  if (!ev.ok) return AR_ERR_HIP;
  for (int i = 0; i < 20; ++i) {
    int rc = decode_once(x, y, w_in, w_out, P, n, 1u, mailbox, flags, d_err, chain, stream);
    if (rc) return rc;
  }
  (void)hipEventRecord(ev.a, s);
  for (int i = 0; i < iters; ++i) {
    int rc = decode_once(x, y, w_in, w_out, P, n, 1u, mailbox, flags, d_err, chain, stream);
    if (rc) return rc;
  }
  (void)hipEventRecord(ev.b, s);
  return ev.us_between(iters);
}

// Decode-size handoff through the waiting unpack.  Handoff i records an
// event on stream sa, packs x with sequence number seq0 + i + 1 on sa, then,
// queued after it, unpacks on stream sb with ar_unpack_fused_wait, which
// polls until its words carry that number (the consumer is launched with no
// dependency on its producer), and records an event on sb.  Handoff i + 1
// waits for handoff i's unpack (it overwrites the words that unpack reads);
// that wait lies between handoffs, outside what is timed.  serial != 0: the
// pack and a plain unpack one after the other on sa.  Returns the median
// microseconds from the first event to the second over `iters` handoffs
// (after 10 untimed ones), or a negative status.
double arb_handoff_us(const void* x, uint64_t* words, void* y, size_t n, uint32_t seq0, uint64_t* d_err,
                      int iters, int serial, void* sa, void* sb) {
  if (iters < 1 || iters > 100000 || !x || !words || !y || !d_err || (!serial && !sb)) return AR_ERR_INVALID;
  hipStream_t a = static_cast<hipStream_t>(sa);
  hipStream_t b = serial ? a : static_cast<hipStream_t>(sb);
  const int total = iters + 10;
  std::vector<hipEvent_t> e0(total, nullptr), e1(total, nullptr);
  int rc = AR_OK;
  for (int i = 0; i < total && rc == AR_OK; ++i)
    if (hipEventCreate(&e0[i]) != hipSuccess || hipEventCreate(&e1[i]) != hipSuccess) rc = AR_ERR_HIP;
  // a delay at the head of both streams (about 7 ms), so every handoff is
  // queued before the GPU reaches it and no host enqueue gap lands between
  // a pair of events
  hipEvent_t head = nullptr;
  if (rc == AR_OK && hipEventCreateWithFlags(&head, hipEventDisableTiming) != hipSuccess) rc = AR_ERR_HIP;
  if (rc == AR_OK) {
    hipLaunchKernelGGL(k_delay, dim3(1), dim3(64), 0, a, 2000);
    if (hipGetLastError() != hipSuccess || hipEventRecord(head, a) != hipSuccess ||
        hipStreamWaitEvent(b, head, 0) != hipSuccess)
      rc = AR_ERR_HIP;
  }
  uint32_t seq = seq0;
  for (int i = 0; i < total && rc == AR_OK; ++i) {
    ++seq;
    if (i > 0 && !serial && hipStreamWaitEvent(a, e1[i - 1], 0) != hipSuccess) rc = AR_ERR_HIP;
    if (rc == AR_OK && hipEventRecord(e0[i], a) != hipSuccess) rc = AR_ERR_HIP;
    if (rc == AR_OK) rc = ar_pack_fused(x, words, n, seq, sa);
    if (rc == AR_OK)
      rc = serial ? ar_unpack_fused(words, y, n, seq, d_err, sa)
                  : ar_unpack_fused_wait(words, y, n, seq, 1u << 20, d_err, sb);
    if (rc == AR_OK && hipEventRecord(e1[i], b) != hipSuccess) rc = AR_ERR_HIP;
  }
  if (hipStreamSynchronize(a) != hipSuccess || hipStreamSynchronize(b) != hipSuccess) rc = rc ? rc : AR_ERR_HIP;
  std::vector<double> us;
  for (int i = 10; i < total && rc == AR_OK; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e0[i], e1[i]) != hipSuccess) rc = AR_ERR_HIP;
    us.push_back(1000.0 * ms);
  }
  for (int i = 0; i < total; ++i) {
    if (e0[i]) (void)hipEventDestroy(e0[i]);
    if (e1[i]) (void)hipEventDestroy(e1[i]);
  }
  if (head) (void)hipEventDestroy(head);
  if (rc != AR_OK) return (double)rc;
  std::nth_element(us.begin(), us.begin() + us.size() / 2, us.end());
  return us[us.size() / 2];
}

// Read-only sweep of `bytes` (a multiple of 16, 16-byte aligned); out holds
// one word per workgroup: ceil(bytes / 16384) words.
int arb_readsum(const void* src, size_t bytes, uint32_t* out, void* stream) {
  if ((bytes & 15u) || !src || !out) return AR_ERR_INVALID;
  const size_t nvec = bytes / 16;
  const size_t grid = (nvec + 1023) / 1024;
  if (grid == 0 || grid > 0x7FFFFFFFull) return AR_ERR_INVALID;
  hipLaunchKernelGGL(k_readsum, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), nvec, out);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
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

// N -> N side-by-side copy (N in {1, 2, 4, 8}) of `bytes` per buffer (a
// multiple of 16; 16-byte aligned buffers), V in {1, 2} groups per lane,
// at most wg_per_cu workgroups per CU through a dynamic LDS request (0: no
// cap).  Buffers must not overlap one another.
int arb_copy_multi(const void* const* ins, void* const* outs, int N, size_t bytes, int vec, int wg_per_cu,
                   void* stream) {
  if (!ins || !outs || (N != 1 && N != 2 && N != 4 && N != 8) || (vec != 1 && vec != 2) ||
      (bytes & 15u) || bytes == 0 || wg_per_cu < 0)
    return AR_ERR_INVALID;
  MultiPtrs m{};
  for (int j = 0; j < N; ++j) {
    if (!ins[j] || !outs[j]) return AR_ERR_INVALID;
    m.in[j] = static_cast<const u32x4*>(ins[j]);
    m.out[j] = static_cast<u32x4*>(outs[j]);
  }
  unsigned lds = 0;
  if (wg_per_cu > 0) {
    int dev = 0, per_cu = 0, per_block = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      return AR_ERR_HIP;
    lds = ((unsigned)per_cu / (unsigned)wg_per_cu) & ~255u;
    if (lds > (unsigned)per_block) lds = (unsigned)per_block;
  }
  const size_t nvec = bytes / 16;
  const size_t grid = (nvec + 64 * (size_t)vec - 1) / (64 * (size_t)vec);
  if (grid > 0x7FFFFFFFull) return AR_ERR_INVALID;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)grid), b(64);
#define ARB_COPY_MULTI(NN)                                                                 \
  if (N == NN) {                                                                           \
    if (vec == 2) hipLaunchKernelGGL((k_copy_multi<NN, 2>), g, b, lds, st, m, nvec);       \
    else hipLaunchKernelGGL((k_copy_multi<NN, 1>), g, b, lds, st, m, nvec);                \
  }
  ARB_COPY_MULTI(1)
  ARB_COPY_MULTI(2)
  ARB_COPY_MULTI(4)
  ARB_COPY_MULTI(8)
#undef ARB_COPY_MULTI
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

// N -> 1 gather (N in {2, 4, 8}): out = XOR of the N inputs, `bytes` per
// buffer (a multiple of 16; 16-byte aligned buffers), non-temporal stores
// when nts != 0, at most wg_per_cu workgroups per CU (0: no cap).  The
// output must not overlap an input.
int arb_gather_xor(const void* const* ins, int N, void* out, size_t bytes, int nts, int wg_per_cu,
                   void* stream) {
  if (!ins || !out || (N != 2 && N != 4 && N != 8) || (bytes & 15u) || bytes == 0 || wg_per_cu < 0)
    return AR_ERR_INVALID;
  MultiPtrs m{};
  for (int j = 0; j < N; ++j) {
    if (!ins[j]) return AR_ERR_INVALID;
    m.in[j] = static_cast<const u32x4*>(ins[j]);
  }
  m.out[0] = static_cast<u32x4*>(out);
  unsigned lds = 0;
  if (wg_per_cu > 0) {
    int dev = 0, per_cu = 0, per_block = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      return AR_ERR_HIP;
    lds = ((unsigned)per_cu / (unsigned)wg_per_cu) & ~255u;
    if (lds > (unsigned)per_block) lds = (unsigned)per_block;
  }
  const size_t nvec = bytes / 16;
  const size_t grid = (nvec + 63) / 64;
  if (grid > 0x7FFFFFFFull) return AR_ERR_INVALID;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)grid), b(64);
#define ARB_GATHER(NN)                                                               \
  if (N == NN) {                                                                     \
    if (nts) hipLaunchKernelGGL((k_gather_xor<NN, true>), g, b, lds, st, m, nvec);   \
    else hipLaunchKernelGGL((k_gather_xor<NN, false>), g, b, lds, st, m, nvec);      \
  }
  ARB_GATHER(2)
  ARB_GATHER(4)
  ARB_GATHER(8)
#undef ARB_GATHER
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

// Launch the chunk consumer (n_elems and chunk_elems multiples of 8, buffers
// 16-byte aligned) with `grid` workgroups of 256 lanes, at most two per CU
// of the current device.  work > 0 adds that many FMA rounds per 16-byte
// group and needs sink (grid * 256 floats).
int arb_consume_chunks(const uint32_t* done, uint32_t epoch, const void* src, void* dst, size_t n_elems,
                       size_t chunk_elems, uint32_t first_chunk, uint32_t max_spins, uint32_t* timeouts,
                       int work, float* sink, int grid, void* stream) {
  if (!done || !src || !dst || !timeouts || (n_elems & 7u) || (chunk_elems & 7u) || chunk_elems == 0 ||
      grid <= 0 || work < 0 || (work > 0 && !sink))
    return AR_ERR_INVALID;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return AR_ERR_HIP;
  if (grid > 2 * cus) return AR_ERR_INVALID;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  if (work > 0)
    hipLaunchKernelGGL(k_consume<true>, dim3(grid), dim3(256), 0, st, done, epoch, s, d, n_elems / 8,
                       chunk_elems / 8, first_chunk, max_spins, timeouts, work, sink);
  else
    hipLaunchKernelGGL(k_consume<false>, dim3(grid), dim3(256), 0, st, done, epoch, s, d, n_elems / 8,
                       chunk_elems / 8, first_chunk, max_spins, timeouts, 0, (float*)nullptr);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

// Launch the ALU stand-in: `grid` workgroups of 256 lanes, out holds grid*256 floats.
int arb_alu(float* out, int iters, int grid, void* stream) {
  if (!out || iters < 0 || grid <= 0) return AR_ERR_INVALID;
  hipLaunchKernelGGL(k_alu, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

}  // extern "C"
