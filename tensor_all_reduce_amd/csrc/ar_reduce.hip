// Reduce kernels for gfx950: one-shot, two-stage (fused write mode and
// staged reduce-scatter / all-gather), and the chunk-major ubatch kernel.
//
// Pages cited (titles as printed):
//   [CAR]    "fix(custom_all_reduce): use SYSTEM scope + ACQUIRE ordering for
//             cross-device signal loads" -- Root cause and Changes 3: the
//             two-stage kernel, whose write mode stores each reduced value
//             straight into every rank's registered output.
//   [NVRAR]  "Technical Summary: Understanding and Improving Communication
//             Performance in Multi-node LLM Inference" -- Methodology 3:
//             reduce-scatter, all-gather; Optimizations: chunked communication.
//   [TBO-AR] "[DSV4] perf(tbo): overlap pure-TP all_reduce on TBO + Delay TP"
//             -- pull request overview: one all-reduce per ubatch on its own
//             stream.
//
// The work is elementwise and HBM-bound: each 16-byte group of 8 bf16 is read
// once from each of the P buffers and written once to each output.  Nothing
// is a contraction, so no MFMA; the kernels aim at bytes in flight: 128-bit
// loads, two groups per lane per iteration (2*P loads issued before the first
// add), grid-stride loops over a grid sized from the CU count.
#include "ar_device.hpp"
#include "ar_internal.hpp"

namespace ar {

// ----------------------------------------------------------------------------
// One-shot (NOUT == 1) and fused two-stage (NOUT == P): grid-stride over the
// 16-byte groups, every group reduced by exactly one lane, so an output that
// is exactly an input buffer is safe (each lane reads its group from every
// input before it writes that group).
template <int P, int NOUT, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void k_reduce(InPtrs in, OutPtrs out, size_t n) {
  const size_t nvec = n >> 3;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const u32x4* src[P];
#pragma unroll
  for (int p = 0; p < P; ++p) src[p] = static_cast<const u32x4*>(in.p[p]);
  u32x4* dst[NOUT];
#pragma unroll
  for (int o = 0; o < NOUT; ++o) dst[o] = static_cast<u32x4*>(out.p[o]);

  for (; v + stride < nvec; v += 2 * stride) {
    u32x4 a[P], b[P];
#pragma unroll
    for (int p = 0; p < P; ++p) a[p] = ld4<NTL>(src[p] + v);
#pragma unroll
    for (int p = 0; p < P; ++p) b[p] = ld4<NTL>(src[p] + v + stride);
    const u32x4 ra = reduce8<P>(a);
#pragma unroll
    for (int o = 0; o < NOUT; ++o) st4<NTS>(dst[o] + v, ra);
    const u32x4 rb = reduce8<P>(b);
#pragma unroll
    for (int o = 0; o < NOUT; ++o) st4<NTS>(dst[o] + v + stride, rb);
  }
  if (v < nvec) {
    u32x4 a[P];
#pragma unroll
    for (int p = 0; p < P; ++p) a[p] = ld4<NTL>(src[p] + v);
    const u32x4 ra = reduce8<P>(a);
#pragma unroll
    for (int o = 0; o < NOUT; ++o) st4<NTS>(dst[o] + v, ra);
  }
  // ragged tail: the last n % 8 elements, one lane each, scalar
  const size_t t0 = nvec << 3;
  if (blockIdx.x == 0 && t0 + threadIdx.x < n) {
    const size_t i = t0 + threadIdx.x;
    const uint16_t* in16[P];
#pragma unroll
    for (int p = 0; p < P; ++p) in16[p] = static_cast<const uint16_t*>(in.p[p]);
    const uint16_t r = reduce1<P>(in16, i);
#pragma unroll
    for (int o = 0; o < NOUT; ++o) static_cast<uint16_t*>(out.p[o])[i] = r;
  }
}

// ----------------------------------------------------------------------------
// Staged two-stage.  Shard s = elements [s*S, min(n, (s+1)*S)), S a multiple
// of 8.  Workgroup b works on shard b % P: workgroups are dispatched to the
// 8 XCDs round-robin, so with P = 8 shard s is reduced (and later gathered)
// by XCD s alone, the one-GPU picture of "rank s owns shard s", and the
// gather re-reads scratch lines through the L2 that wrote them.
template <int P, bool NTL>
__global__ __launch_bounds__(kBlock) void k_rs(InPtrs in, void* scratch, size_t n, size_t S) {
  const unsigned s = blockIdx.x % P;
  const unsigned j = blockIdx.x / P;
  const unsigned bps = gridDim.x / P;
  const size_t lo = (size_t)s * S < n ? (size_t)s * S : n;
  const size_t hi = lo + S < n ? lo + S : n;
  const size_t vlo = lo >> 3, vhi = hi >> 3;
  const size_t stride = (size_t)bps * blockDim.x;
  const u32x4* src[P];
#pragma unroll
  for (int p = 0; p < P; ++p) src[p] = static_cast<const u32x4*>(in.p[p]);
  u32x4* dst = static_cast<u32x4*>(scratch);
  size_t v = vlo + (size_t)j * blockDim.x + threadIdx.x;
  for (; v + stride < vhi; v += 2 * stride) {
    u32x4 a[P], b[P];
#pragma unroll
    for (int p = 0; p < P; ++p) a[p] = ld4<NTL>(src[p] + v);
#pragma unroll
    for (int p = 0; p < P; ++p) b[p] = ld4<NTL>(src[p] + v + stride);
    dst[v] = reduce8<P>(a);
    dst[v + stride] = reduce8<P>(b);
  }
  if (v < vhi) {
    u32x4 a[P];
#pragma unroll
    for (int p = 0; p < P; ++p) a[p] = ld4<NTL>(src[p] + v);
    dst[v] = reduce8<P>(a);
  }
  if (j == 0 && (vhi << 3) + threadIdx.x < hi) {
    const size_t i = (vhi << 3) + threadIdx.x;
    const uint16_t* in16[P];
#pragma unroll
    for (int p = 0; p < P; ++p) in16[p] = static_cast<const uint16_t*>(in.p[p]);
    static_cast<uint16_t*>(scratch)[i] = reduce1<P>(in16, i);
  }
}

template <int P, bool NTS>
__global__ __launch_bounds__(kBlock) void k_ag(const void* scratch, OutPtrs out, size_t n, size_t S) {
  const unsigned s = blockIdx.x % P;
  const unsigned j = blockIdx.x / P;
  const unsigned bps = gridDim.x / P;
  const size_t lo = (size_t)s * S < n ? (size_t)s * S : n;
  const size_t hi = lo + S < n ? lo + S : n;
  const size_t vlo = lo >> 3, vhi = hi >> 3;
  const size_t stride = (size_t)bps * blockDim.x;
  const u32x4* src = static_cast<const u32x4*>(scratch);
  u32x4* dst[P];
#pragma unroll
  for (int p = 0; p < P; ++p) dst[p] = static_cast<u32x4*>(out.p[p]);
  size_t v = vlo + (size_t)j * blockDim.x + threadIdx.x;
  for (; v + stride < vhi; v += 2 * stride) {
    const u32x4 a = src[v];
    const u32x4 b = src[v + stride];
#pragma unroll
    for (int p = 0; p < P; ++p) st4<NTS>(dst[p] + v, a);
#pragma unroll
    for (int p = 0; p < P; ++p) st4<NTS>(dst[p] + v + stride, b);
  }
  if (v < vhi) {
    const u32x4 a = src[v];
#pragma unroll
    for (int p = 0; p < P; ++p) st4<NTS>(dst[p] + v, a);
  }
  if (j == 0 && (vhi << 3) + threadIdx.x < hi) {
    const size_t i = (vhi << 3) + threadIdx.x;
    const uint16_t r = static_cast<const uint16_t*>(scratch)[i];
#pragma unroll
    for (int p = 0; p < P; ++p) static_cast<uint16_t*>(out.p[p])[i] = r;
  }
}

// ----------------------------------------------------------------------------
// Chunk-major reduce of elements [e0, e1).  Chunk c covers
// [e0 + c*chunk, min(e0 + (c+1)*chunk, e1)); workgroup b handles slice
// b % bpc of chunk b / bpc, so workgroups are dispatched in ascending chunk
// order and no workgroup straddles a chunk boundary.  Each slice is up to
// kChunkU * blockDim * 8 elements; misaligned slice ends (when e0 or the
// chunk length is not a multiple of 8) are done element by element.
constexpr int kChunkU = 2;

template <int P, int NOUT, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void k_chunk(InPtrs in, OutPtrs out, size_t e0, size_t e1,
                                                  size_t chunk, unsigned bpc) {
  const size_t c = blockIdx.x / bpc;
  const unsigned t = blockIdx.x % bpc;
  const size_t span = (size_t)kChunkU * blockDim.x * 8;
  const size_t c0 = e0 + c * chunk;
  const size_t c1 = c0 + chunk < e1 ? c0 + chunk : e1;
  const size_t b0 = c0 + (size_t)t * span;
  if (b0 >= c1) return;
  const size_t b1 = b0 + span < c1 ? b0 + span : c1;
  const size_t vb0 = (b0 + 7) >> 3, vb1 = b1 >> 3;

  const u32x4* src[P];
#pragma unroll
  for (int p = 0; p < P; ++p) src[p] = static_cast<const u32x4*>(in.p[p]);
  u32x4 x[kChunkU][P];
  bool ok[kChunkU];
#pragma unroll
  for (int u = 0; u < kChunkU; ++u) {
    const size_t v = vb0 + threadIdx.x + (size_t)u * blockDim.x;
    ok[u] = v < vb1;
    if (ok[u]) {
#pragma unroll
      for (int p = 0; p < P; ++p) x[u][p] = ld4<NTL>(src[p] + v);
    }
  }
#pragma unroll
  for (int u = 0; u < kChunkU; ++u) {
    if (ok[u]) {
      const size_t v = vb0 + threadIdx.x + (size_t)u * blockDim.x;
      const u32x4 r = reduce8<P>(x[u]);
#pragma unroll
      for (int o = 0; o < NOUT; ++o) st4<NTS>(static_cast<u32x4*>(out.p[o]) + v, r);
    }
  }
  // element-wise head [b0, min(8*vb0, b1)) and tail [max(8*vb1, 8*vb0), b1)
  const size_t h1 = (vb0 << 3) < b1 ? (vb0 << 3) : b1;
  const size_t t0 = (vb1 > vb0 ? vb1 : vb0) << 3;
  size_t i = b0 + threadIdx.x;
  if (i >= h1) i = t0 + (i - h1);
  if (i < b1 && (i < h1 || i >= t0)) {
    const uint16_t* in16[P];
#pragma unroll
    for (int p = 0; p < P; ++p) in16[p] = static_cast<const uint16_t*>(in.p[p]);
    const uint16_t r = reduce1<P>(in16, i);
#pragma unroll
    for (int o = 0; o < NOUT; ++o) static_cast<uint16_t*>(out.p[o])[i] = r;
  }
}

// ----------------------------------------------------------------------------
// Host-side dispatch: P and the non-temporal choices are template
// parameters, so every instantiation has straight-line per-rank code.

namespace {

// Grid for the grid-stride kernels: enough workgroups to give every lane one
// group when the message is small (latency regime), capped at cus*grid_mult
// for large messages (each lane then loops).
inline unsigned stream_grid(const Launch& L, size_t nvec) {
  const size_t want = cdiv(nvec, kBlock);
  const size_t cap = (size_t)L.cus * (size_t)L.grid_mult;
  size_t g = want < cap ? want : cap;
  return (unsigned)(g ? g : 1);
}

template <int P, int NOUT>
hipError_t reduce_p(const Launch& L, const InPtrs& in, const OutPtrs& out, size_t n) {
  const unsigned g = stream_grid(L, n >> 3);
  const int m = (L.nt_loads ? 1 : 0) | (L.nt_stores ? 2 : 0);
  switch (m) {
    case 0: return launch_k(k_reduce<P, NOUT, false, false>, g, kBlock, L.stream, in, out, n);
    case 1: return launch_k(k_reduce<P, NOUT, true, false>, g, kBlock, L.stream, in, out, n);
    case 2: return launch_k(k_reduce<P, NOUT, false, true>, g, kBlock, L.stream, in, out, n);
    default: return launch_k(k_reduce<P, NOUT, true, true>, g, kBlock, L.stream, in, out, n);
  }
}

template <int P>
hipError_t staged_p(const Launch& L, const InPtrs& in, const OutPtrs& out, size_t n, void* scratch) {
  const size_t groups = cdiv(n, 8);
  const size_t S = cdiv(groups, P) * 8;
  const size_t shard_vec = S / 8;
  size_t bps = cdiv(shard_vec, kBlock);
  const size_t cap = cdiv((size_t)L.cus * (size_t)L.grid_mult, P);
  if (bps > cap) bps = cap;
  if (bps == 0) bps = 1;
  const unsigned g = (unsigned)(bps * P);
  hipError_t e = L.nt_loads ? launch_k(k_rs<P, true>, g, kBlock, L.stream, in, scratch, n, S)
                            : launch_k(k_rs<P, false>, g, kBlock, L.stream, in, scratch, n, S);
  if (e != hipSuccess) return e;
  return L.nt_stores ? launch_k(k_ag<P, true>, g, kBlock, L.stream, (const void*)scratch, out, n, S)
                     : launch_k(k_ag<P, false>, g, kBlock, L.stream, (const void*)scratch, out, n, S);
}

template <int P, int NOUT>
hipError_t chunk_p(const Launch& L, const InPtrs& in, const OutPtrs& out, size_t e0, size_t e1,
                   size_t chunk) {
  const size_t span = (size_t)kChunkU * kBlock * 8;
  const size_t bpc = cdiv(chunk, span);
  const size_t nchunks = cdiv(e1 - e0, chunk);
  const size_t blocks = nchunks * bpc;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
  const int m = (L.nt_loads ? 1 : 0) | (L.nt_stores ? 2 : 0);
  const unsigned g = (unsigned)blocks, b = (unsigned)bpc;
  switch (m) {
    case 0: return launch_k(k_chunk<P, NOUT, false, false>, g, kBlock, L.stream, in, out, e0, e1, chunk, b);
    case 1: return launch_k(k_chunk<P, NOUT, true, false>, g, kBlock, L.stream, in, out, e0, e1, chunk, b);
    case 2: return launch_k(k_chunk<P, NOUT, false, true>, g, kBlock, L.stream, in, out, e0, e1, chunk, b);
    default: return launch_k(k_chunk<P, NOUT, true, true>, g, kBlock, L.stream, in, out, e0, e1, chunk, b);
  }
}

}  // namespace

#define AR_DISPATCH_P(P, EXPR_T)                     \
  switch (P) {                                       \
    case 1: { constexpr int PP = 1; return EXPR_T; } \
    case 2: { constexpr int PP = 2; return EXPR_T; } \
    case 3: { constexpr int PP = 3; return EXPR_T; } \
    case 4: { constexpr int PP = 4; return EXPR_T; } \
    case 5: { constexpr int PP = 5; return EXPR_T; } \
    case 6: { constexpr int PP = 6; return EXPR_T; } \
    case 7: { constexpr int PP = 7; return EXPR_T; } \
    case 8: { constexpr int PP = 8; return EXPR_T; } \
    default: return hipErrorInvalidValue;            \
  }

hipError_t launch_oneshot(const Launch& L, const InPtrs& in, int P, void* out, size_t n) {
  OutPtrs o{};
  o.p[0] = out;
  AR_DISPATCH_P(P, (reduce_p<PP, 1>(L, in, o, n)))
}

hipError_t launch_2stage_fused(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                               size_t n) {
  AR_DISPATCH_P(P, (reduce_p<PP, PP>(L, in, out, n)))
}

hipError_t launch_2stage_staged(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                                size_t n, void* scratch) {
  AR_DISPATCH_P(P, (staged_p<PP>(L, in, out, n, scratch)))
}

hipError_t launch_chunked(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                          size_t e0, size_t e1, size_t chunk_elems, int two_stage) {
  if (two_stage) {
    AR_DISPATCH_P(P, (chunk_p<PP, PP>(L, in, out, e0, e1, chunk_elems)))
  }
  AR_DISPATCH_P(P, (chunk_p<PP, 1>(L, in, out, e0, e1, chunk_elems)))
}

}  // namespace ar
