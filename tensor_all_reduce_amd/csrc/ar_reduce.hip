// Reduce kernels for gfx950: one-shot, two-stage (fused write mode and
// staged reduce-scatter / all-gather) and the chunked ubatch reduce.
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
// once from each of the P buffers and written once to each output; no MFMA.
// Launch shape (chosen by measurement on MI355X; the per-kernel table lives
// in the API layer): a flat grid of small workgroups, each owning one
// contiguous tile of V * blockDim groups, one group per lane per pass.
// Workgroups are dispatched in index order, so the tiles in flight form a
// compact, advancing window of each buffer; a persistent grid-stride loop
// spreads the in-flight accesses over the whole buffer and measured up to
// 20% slower.  Workgroups per CU are capped per kernel (see Shape).
#include "ar_device.hpp"
#include "ar_internal.hpp"

namespace ar {

// ----------------------------------------------------------------------------
// Range reduce over elements [e0, e1) of every buffer, chunk-major.
// Chunk c covers [e0 + c*chunk, min(e0 + (c+1)*chunk, e1)); workgroup b works
// on tile b % bpc of chunk b / bpc, so tiles never straddle a chunk boundary
// and chunks are dispatched in ascending order.  A whole-buffer reduce is the
// single-chunk case.  Tiles are V * blockDim groups of 8 elements; groups are
// aligned to the buffer base, and a tile end that falls inside a group (e0 or
// the chunk length not a multiple of 8, or the ragged end of the buffer) is
// done element by element.  NOUT == 1: one-shot; NOUT == P: fused two-stage
// (write mode).  Every group is reduced by exactly one lane, which reads it
// from every input before writing it, so an output equal to an input is safe.
//
// SIG: the workgroups of a chunk also publish its completion.  Every output
// store is device-coherent (written through past the XCD's L2), each wave
// waits until its stores are acknowledged, the workgroup meets at a barrier,
// and one lane adds 1 to the chunk's tile counter; the workgroup that
// completes the count resets the counter to zero (ready for the next call)
// and stores sig.epoch into done[chunk].  This is an agent-scope release
// without the L2 writeback: nothing the flag covers was left dirty in an L2.
// The flag store depends on the counter's returned value, and every counter
// increment follows its workgroup's acknowledged stores, so a consumer that
// acquire-loads done[chunk] == epoch (which invalidates its own L2 and L1
// copies) sees the whole chunk of every output.
template <int P, int NOUT, int V, bool NTL, bool NTS, bool SIG>
__global__ __launch_bounds__(kMaxBlock) void k_reduce(InPtrs in, OutPtrs out, size_t e0, size_t e1,
                                                     size_t chunk, unsigned bpc, ChunkSignal sig) {
  const size_t span = (size_t)V * blockDim.x * 8;
  const size_t c = blockIdx.x / bpc;
  const unsigned t = blockIdx.x % bpc;
  const size_t c0 = e0 + c * chunk;
  const size_t c1 = c0 + chunk < e1 ? c0 + chunk : e1;
  const size_t b0 = c0 + (size_t)t * span;
  if (b0 >= c1) return;
  const size_t b1 = b0 + span < c1 ? b0 + span : c1;
  const size_t vb0 = (b0 + 7) >> 3, vb1 = b1 >> 3;

  u32x4 x[V][P];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t v = vb0 + threadIdx.x + (size_t)u * blockDim.x;
    if (v < vb1) {
#pragma unroll
      for (int p = 0; p < P; ++p) x[u][p] = ld4<NTL>(static_cast<const u32x4*>(in.p[p]) + v);
    }
  }
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t v = vb0 + threadIdx.x + (size_t)u * blockDim.x;
    if (v < vb1) {
      const u32x4 r = reduce8<P>(x[u]);
#pragma unroll
      for (int o = 0; o < NOUT; ++o) {
        if constexpr (SIG)
          st4_coherent<NTS>(static_cast<u32x4*>(out.p[o]) + vb0, (uint32_t)((vb1 - vb0) * 16),
                            (uint32_t)((v - vb0) * 16), r);
        else
          st4<NTS>(static_cast<u32x4*>(out.p[o]) + v, r);
      }
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
    for (int o = 0; o < NOUT; ++o) {
      uint16_t* dst = static_cast<uint16_t*>(out.p[o]) + i;
      if constexpr (SIG) __hip_atomic_store(dst, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *dst = r;
    }
  }
  if constexpr (SIG) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned g = sig.base + (unsigned)c;
      const unsigned tiles_here = (unsigned)((c1 - c0 + span - 1) / span);
      const unsigned old = __hip_atomic_fetch_add(sig.tiles + g, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1u == tiles_here) {
        __hip_atomic_store(sig.tiles + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(sig.done + g, sig.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Staged two-stage.  Shard s = elements [s*S, min(n, (s+1)*S)), S a multiple
// of 8.  Workgroup b works on tile b / P of shard b % P: workgroups go to the
// 8 XCDs round-robin, so with P = 8 shard s is reduced (and later gathered)
// by XCD s alone -- the one-GPU picture of "rank s owns shard s" -- and the
// gather re-reads scratch lines through the L2 that wrote them.
template <int P, bool NTL>
__global__ __launch_bounds__(kMaxBlock) void k_rs(InPtrs in, void* scratch, size_t n, size_t S) {
  const unsigned s = blockIdx.x % P;
  const size_t j = blockIdx.x / P;
  const size_t lo = (size_t)s * S < n ? (size_t)s * S : n;
  const size_t hi = lo + S < n ? lo + S : n;
  const size_t v = (lo >> 3) + j * blockDim.x + threadIdx.x;
  if (v < (hi >> 3)) {
    u32x4 a[P];
#pragma unroll
    for (int p = 0; p < P; ++p) a[p] = ld4<NTL>(static_cast<const u32x4*>(in.p[p]) + v);
    static_cast<u32x4*>(scratch)[v] = reduce8<P>(a);
  }
  if (j == 0 && ((hi >> 3) << 3) + threadIdx.x < hi) {
    const size_t i = ((hi >> 3) << 3) + threadIdx.x;
    const uint16_t* in16[P];
#pragma unroll
    for (int p = 0; p < P; ++p) in16[p] = static_cast<const uint16_t*>(in.p[p]);
    static_cast<uint16_t*>(scratch)[i] = reduce1<P>(in16, i);
  }
}

template <int P, bool NTS>
__global__ __launch_bounds__(kMaxBlock) void k_ag(const void* scratch, OutPtrs out, size_t n, size_t S) {
  const unsigned s = blockIdx.x % P;
  const size_t j = blockIdx.x / P;
  const size_t lo = (size_t)s * S < n ? (size_t)s * S : n;
  const size_t hi = lo + S < n ? lo + S : n;
  const size_t v = (lo >> 3) + j * blockDim.x + threadIdx.x;
  if (v < (hi >> 3)) {
    const u32x4 a = static_cast<const u32x4*>(scratch)[v];
#pragma unroll
    for (int p = 0; p < P; ++p) st4<NTS>(static_cast<u32x4*>(out.p[p]) + v, a);
  }
  if (j == 0 && ((hi >> 3) << 3) + threadIdx.x < hi) {
    const size_t i = ((hi >> 3) << 3) + threadIdx.x;
    const uint16_t r = static_cast<const uint16_t*>(scratch)[i];
#pragma unroll
    for (int p = 0; p < P; ++p) static_cast<uint16_t*>(out.p[p])[i] = r;
  }
}

// ----------------------------------------------------------------------------
namespace {

template <int P, int NOUT, int V>
hipError_t range_v(const Shape& sh, hipStream_t st, const InPtrs& in, const OutPtrs& out, size_t e0,
                   size_t e1, size_t chunk, const ChunkSignal& sig) {
  const size_t span = (size_t)V * sh.block * 8;
  const size_t bpc = cdiv(chunk, span);
  const size_t nchunks = cdiv(e1 - e0, chunk);
  const size_t blocks = nchunks * bpc;
  if (blocks > 0x7FFFFFFFull || bpc > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
  const unsigned g = (unsigned)blocks, b = (unsigned)bpc;
  const dim3 blk(sh.block);
  if (sig.done != nullptr) {
    if (sh.nt_loads && sh.nt_stores)
      return launch_k(k_reduce<P, NOUT, V, true, true, true>, g, blk, sh.lds, st, in, out, e0, e1, chunk, b, sig);
    if (sh.nt_loads)
      return launch_k(k_reduce<P, NOUT, V, true, false, true>, g, blk, sh.lds, st, in, out, e0, e1, chunk, b, sig);
    if (sh.nt_stores)
      return launch_k(k_reduce<P, NOUT, V, false, true, true>, g, blk, sh.lds, st, in, out, e0, e1, chunk, b, sig);
    return launch_k(k_reduce<P, NOUT, V, false, false, true>, g, blk, sh.lds, st, in, out, e0, e1, chunk, b, sig);
  }
  if (sh.nt_loads && sh.nt_stores)
    return launch_k(k_reduce<P, NOUT, V, true, true, false>, g, blk, sh.lds, st, in, out, e0, e1, chunk, b, sig);
  if (sh.nt_loads)
    return launch_k(k_reduce<P, NOUT, V, true, false, false>, g, blk, sh.lds, st, in, out, e0, e1, chunk, b, sig);
  if (sh.nt_stores)
    return launch_k(k_reduce<P, NOUT, V, false, true, false>, g, blk, sh.lds, st, in, out, e0, e1, chunk, b, sig);
  return launch_k(k_reduce<P, NOUT, V, false, false, false>, g, blk, sh.lds, st, in, out, e0, e1, chunk, b, sig);
}

template <int P, int NOUT>
hipError_t range_p(const Shape& sh, hipStream_t st, const InPtrs& in, const OutPtrs& out, size_t e0,
                   size_t e1, size_t chunk, const ChunkSignal& sig = ChunkSignal{nullptr, nullptr, 0, 0}) {
  if (sh.vec == 2) return range_v<P, NOUT, 2>(sh, st, in, out, e0, e1, chunk, sig);
  return range_v<P, NOUT, 1>(sh, st, in, out, e0, e1, chunk, sig);
}

template <int P>
hipError_t staged_p(const Launch& L, const InPtrs& in, const OutPtrs& out, size_t n, void* scratch) {
  const size_t S = cdiv(cdiv(n, 8), P) * 8;
  const Shape& rs = L.shape[kRS];
  const Shape& ag = L.shape[kAG];
  const size_t bps_rs = cdiv(S / 8, (size_t)rs.block), bps_ag = cdiv(S / 8, (size_t)ag.block);
  if (bps_rs * P > 0x7FFFFFFFull || bps_ag * P > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
  const unsigned g_rs = (unsigned)(bps_rs * P), g_ag = (unsigned)(bps_ag * P);
  hipError_t e = rs.nt_loads
                     ? launch_k(k_rs<P, true>, g_rs, dim3(rs.block), rs.lds, L.stream, in, scratch, n, S)
                     : launch_k(k_rs<P, false>, g_rs, dim3(rs.block), rs.lds, L.stream, in, scratch, n, S);
  if (e != hipSuccess) return e;
  return ag.nt_stores ? launch_k(k_ag<P, true>, g_ag, dim3(ag.block), ag.lds, L.stream,
                                 (const void*)scratch, out, n, S)
                      : launch_k(k_ag<P, false>, g_ag, dim3(ag.block), ag.lds, L.stream,
                                 (const void*)scratch, out, n, S);
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
  AR_DISPATCH_P(P, (range_p<PP, 1>(shape_for(L, kOneshot, kOneshotSmall, n), L.stream, in, o, 0, n, n)))
}

hipError_t launch_2stage_fused(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                               size_t n) {
  AR_DISPATCH_P(P, (range_p<PP, PP>(shape_for(L, k2Stage, k2StageSmall, n), L.stream, in, out, 0, n, n)))
}

hipError_t launch_2stage_staged(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                                size_t n, void* scratch) {
  AR_DISPATCH_P(P, (staged_p<PP>(L, in, out, n, scratch)))
}

hipError_t launch_chunked(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                          size_t e0, size_t e1, size_t chunk_elems, int two_stage,
                          const ChunkSignal& sig) {
  // the flagged variant has its own shape: every workgroup of a chunk waits
  // for its stores and adds to a counter, so fewer, larger workgroups are
  // cheaper (256 lanes: the wait is hidden by the other waves)
  const Shape& sh2 = sig.done ? L.shape[kUbatchFlags] : L.shape[kUbatch];
  const Shape& sh1 = sig.done ? L.shape[kUbatchFlags] : L.shape[kOneshot];
  if (two_stage) {
    AR_DISPATCH_P(P, (range_p<PP, PP>(sh2, L.stream, in, out, e0, e1, chunk_elems, sig)))
  }
  AR_DISPATCH_P(P, (range_p<PP, 1>(sh1, L.stream, in, out, e0, e1, chunk_elems, sig)))
}

}  // namespace ar
