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
#include "ar_offsets.hpp"

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
// Outputs are stored with policy SP (st16).  SIG: the workgroups of a chunk
// also publish its completion.  Every output store is then device-coherent
// (SP is 2 or 3: written through past the XCD's L2), each wave
// waits until its stores are acknowledged, the workgroup meets at a barrier,
// and one lane adds 1 to the chunk's tile counter; the workgroup that
// completes the count resets the counter to zero (ready for the next call)
// and stores sig.epoch into done[chunk].  This is an agent-scope release
// without the L2 writeback: nothing the flag covers was left dirty in an L2.
// The flag store depends on the counter's returned value, and every counter
// increment follows its workgroup's acknowledged stores, so a consumer that
// acquire-loads done[chunk] == epoch (which invalidates its own L2 and L1
// copies) sees the whole chunk of every output.
//
// `nthr` is the workgroup size (blockDim.x, or a compile-time constant where
// the kernel must not read the dispatch's hidden arguments).
template <int P, int NOUT, int V, bool NTL, int SP, bool SIG>
__device__ __forceinline__ void reduce_tile(const InPtrs& in, const OutPtrs& out, size_t b0, size_t b1,
                                            unsigned nthr) {
  const size_t vb0 = (b0 + 7) >> 3, vb1 = b1 >> 3;
  static_assert(!SIG || SP >= 2, "completion flags need write-through stores");

  u32x4 x[V][P];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t v = vb0 + threadIdx.x + (size_t)u * nthr;
    if (v < vb1) {
#pragma unroll
      for (int p = 0; p < P; ++p) x[u][p] = ld4<NTL>(static_cast<const u32x4*>(in.p[p]) + v);
    }
  }
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t v = vb0 + threadIdx.x + (size_t)u * nthr;
    if (v < vb1) {
      const u32x4 r = reduce8<P>(x[u]);
#pragma unroll
      for (int o = 0; o < NOUT; ++o)
        st16<SP>(static_cast<u32x4*>(out.p[o]) + vb0, (uint32_t)((vb1 - vb0) * 16), (uint32_t)((v - vb0) * 16), r);
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
}

template <int P, int NOUT, int V, bool NTL, int SP, bool SIG>
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
  reduce_tile<P, NOUT, V, NTL, SP, SIG>(in, out, b0, b1, blockDim.x);
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

// Bounded-footprint range reduce: the same tiles, in the same chunk-major
// order, as k_reduce, but a persistent grid of gridDim.x workgroups walks
// them (workgroup w takes tiles w, w + G, w + 2G, ...), so the reduce holds
// only that many workgroup slots -- with one large workgroup per CU, a
// fraction of the CUs -- and leaves the rest of the device to compute
// running beside it on another stream (the partner ubatch of [TBO-AR]).  At
// any moment the grid's tiles form one compact window that advances through
// the chunks in ascending order.  Every tile is reduced exactly as k_reduce
// reduces it, so the results are identical.
template <int P, int NOUT, int V, bool NTL, int SP>
__global__ __launch_bounds__(kMaxBlockBounded) void k_reduce_bounded(InPtrs in, OutPtrs out, size_t e0,
                                                                    size_t e1, size_t chunk, unsigned bpc,
                                                                    size_t ntiles) {
  const size_t span = (size_t)V * blockDim.x * 8;
  for (size_t g = blockIdx.x; g < ntiles; g += gridDim.x) {
    const size_t c = g / bpc;
    const size_t t = g - c * bpc;
    const size_t c0 = e0 + c * chunk;
    const size_t c1 = c0 + chunk < e1 ? c0 + chunk : e1;
    const size_t b0 = c0 + t * span;
    if (b0 >= c1) continue;
    const size_t b1 = b0 + span < c1 ? b0 + span : c1;
    reduce_tile<P, NOUT, V, NTL, SP, false>(in, out, b0, b1, blockDim.x);
  }
}

// ----------------------------------------------------------------------------
// One-shot for small messages (n <= AR_SMALL_ELEMS) with a compact kernel
// argument segment: the input pointers, the output and n, 80 bytes, and no
// hidden arguments (the workgroup size is the template constant BLOCK, so the
// kernel never reads blockDim).  A decode-size one-shot is bound by the
// host's cost of enqueueing it, and HIP enqueues a kernel whose argument
// segment is at most 112 bytes about 0.7 us faster than a larger one;
// k_reduce's segment is 440 bytes (its chunk and signal arguments, then the
// hidden arguments that reading blockDim brings).  One group per lane; the
// tiles, and so the results, are k_reduce's with a single chunk.
//
// The grid is cdiv(n, 8 * BLOCK), so every workgroup's tile starts below n;
// the compact kernels have no early exit on b0 >= n (where reduce_tile would
// touch nothing anyway), so that the compiler loads n and the buffer
// pointers from the argument segment together instead of one after the
// other.
template <int P, int BLOCK, bool NTL, int SP>
__global__ __launch_bounds__(BLOCK) void k_oneshot_small(InPtrs in, void* out, size_t n) {
  constexpr size_t span = (size_t)BLOCK * 8;
  const size_t b0 = (size_t)blockIdx.x * span;
  const size_t b1 = b0 + span < n ? b0 + span : n;
  OutPtrs o{};
  o.p[0] = out;
  reduce_tile<P, 1, 1, NTL, SP, false>(in, o, b0, b1, BLOCK);
}

// In-place fused two-stage for small messages: every output is its own input
// (the all-reduce's usual form, each rank's result in its own tensor), so
// the P buffer pointers and n, 72 bytes, are the whole argument segment --
// under HIP's fast-enqueue size, as for k_oneshot_small.  Each group is read
// from every buffer by one lane before that lane writes it back to all of
// them, so reading and writing the same buffers is safe.
template <int P, int BLOCK, bool NTL, int SP>
__global__ __launch_bounds__(BLOCK) void k_2stage_small_inplace(OutPtrs io, size_t n) {
  constexpr size_t span = (size_t)BLOCK * 8;
  const size_t b0 = (size_t)blockIdx.x * span;
  const size_t b1 = b0 + span < n ? b0 + span : n;
  InPtrs in;
#pragma unroll
  for (int p = 0; p < AR_MAX_RANKS; ++p) in.p[p] = io.p[p];
  reduce_tile<P, P, 1, NTL, SP, false>(in, io, b0, b1, BLOCK);
}

// Fused two-stage for small messages with separate outputs: ins[0] and the
// other 2P - 1 buffers as 32-bit offsets from it (PtrOffsets, built on the
// host by pack_offsets), an 80-byte argument segment instead of 136 bytes.
template <int P, int BLOCK, bool NTL, int SP>
__global__ __launch_bounds__(BLOCK) void k_2stage_small_offs(PtrOffsets po, size_t n) {
  constexpr size_t span = (size_t)BLOCK * 8;
  const size_t b0 = (size_t)blockIdx.x * span;
  const size_t b1 = b0 + span < n ? b0 + span : n;
  InPtrs in{};
  OutPtrs out{};
  in.p[0] = po.base;
#pragma unroll
  for (int p = 1; p < P; ++p) in.p[p] = offset_address(po, p - 1);
#pragma unroll
  for (int o = 0; o < P; ++o) out.p[o] = const_cast<char*>(offset_address(po, P - 1 + o));
  reduce_tile<P, P, 1, NTL, SP, false>(in, out, b0, b1, BLOCK);
}

// ----------------------------------------------------------------------------
// Staged two-stage.  Shard s = elements [s*S, min(n, (s+1)*S)), S a multiple
// of 8.  Workgroup b works on tile b / P of shard b % P: workgroups go to the
// 8 XCDs round-robin, so with P = 8 shard s is reduced (and later gathered)
// by XCD s alone -- the one-GPU picture of "rank s owns shard s" -- and the
// gather re-reads scratch lines through the L2 that wrote them.
//
// The ragged tail (n not a multiple of 8) lies in the last non-empty shard;
// trailing shards past it are empty (lo == hi == n) and do nothing, so the
// tail elements are written by one workgroup only.  An empty shard's group
// range is empty by itself (v >= n / 8), so only the tail write tests
// lo < hi: with no early exit the compiler loads every argument at once
// instead of the shard bounds first and the pointers after them.
//
// The workgroup size is the template constant BLOCK (64, 128 or 256), so the
// kernels read no hidden dispatch arguments: their argument segments are 88
// bytes, under the size that HIP enqueues about 0.7 us faster, which is what
// a decode-size staged call made from the host waits on (two launches).
template <int P, int BLOCK, bool NTL, int SP>
__global__ __launch_bounds__(BLOCK) void k_rs(InPtrs in, void* scratch, size_t n, size_t S) {
  const unsigned s = blockIdx.x % P;
  const size_t j = blockIdx.x / P;
  const size_t lo = (size_t)s * S < n ? (size_t)s * S : n;
  const size_t hi = lo + S < n ? lo + S : n;
  const size_t w0 = (lo >> 3) + j * BLOCK;  // this workgroup's first group
  const size_t v = w0 + threadIdx.x;
  if (v < (hi >> 3)) {
    u32x4 a[P];
#pragma unroll
    for (int p = 0; p < P; ++p) a[p] = ld4<NTL>(static_cast<const u32x4*>(in.p[p]) + v);
    st16<SP>(static_cast<u32x4*>(scratch) + w0, BLOCK * 16u, threadIdx.x * 16u, reduce8<P>(a));
  }
  if (j == 0 && lo < hi && ((hi >> 3) << 3) + threadIdx.x < hi) {
    const size_t i = ((hi >> 3) << 3) + threadIdx.x;
    const uint16_t* in16[P];
#pragma unroll
    for (int p = 0; p < P; ++p) in16[p] = static_cast<const uint16_t*>(in.p[p]);
    static_cast<uint16_t*>(scratch)[i] = reduce1<P>(in16, i);
  }
}

template <int P, int BLOCK, bool NTL, int SP>
__global__ __launch_bounds__(BLOCK) void k_ag(const void* scratch, OutPtrs out, size_t n, size_t S) {
  const unsigned s = blockIdx.x % P;
  const size_t j = blockIdx.x / P;
  const size_t lo = (size_t)s * S < n ? (size_t)s * S : n;
  const size_t hi = lo + S < n ? lo + S : n;
  const size_t w0 = (lo >> 3) + j * BLOCK;
  const size_t v = w0 + threadIdx.x;
  if (v < (hi >> 3)) {
    const u32x4 a = ld4<NTL>(static_cast<const u32x4*>(scratch) + v);
#pragma unroll
    for (int p = 0; p < P; ++p) st16<SP>(static_cast<u32x4*>(out.p[p]) + w0, BLOCK * 16u, threadIdx.x * 16u, a);
  }
  if (j == 0 && lo < hi && ((hi >> 3) << 3) + threadIdx.x < hi) {
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
  if (sig.done != nullptr) {  // flagged: write-through stores (SC1), NT hint from the shape
    auto go = [&](auto ntl, auto sp) {
      return launch_k(k_reduce<P, NOUT, V, decltype(ntl)::value, decltype(sp)::value, true>, g, blk, sh.lds, st,
                      in, out, e0, e1, chunk, b, sig);
    };
    const bool nt = (sh.stores & 1) != 0;
    if (sh.nt_loads) return nt ? go(std::true_type{}, SPc<3>{}) : go(std::true_type{}, SPc<2>{});
    return nt ? go(std::false_type{}, SPc<3>{}) : go(std::false_type{}, SPc<2>{});
  }
  return with_policy(sh, [&](auto ntl, auto sp) {
    return launch_k(k_reduce<P, NOUT, V, decltype(ntl)::value, decltype(sp)::value, false>, g, blk, sh.lds, st,
                    in, out, e0, e1, chunk, b, sig);
  });
}

// Bounded grid: cus * wg_per_cu / 8 workgroups (wg_per_cu counts eighths of
// the device), at least one and no more than there are tiles.
inline size_t bounded_grid(const Shape& sh, int cus, size_t ntiles) {
  size_t g = (size_t)cus * (size_t)(sh.wg_per_cu > 0 ? sh.wg_per_cu : 8) / 8;
  if (g < 1) g = 1;
  return g < ntiles ? g : ntiles;
}

template <int P, int NOUT, int V>
hipError_t bounded_v(const Shape& sh, int cus, hipStream_t st, const InPtrs& in, const OutPtrs& out, size_t e0,
                     size_t e1, size_t chunk) {
  const size_t span = (size_t)V * sh.block * 8;
  const size_t bpc = cdiv(chunk, span);
  const size_t nchunks = cdiv(e1 - e0, chunk);
  if (bpc > 0xFFFFFFFFull || nchunks > (~(size_t)0) / bpc) return hipErrorInvalidConfiguration;
  const size_t ntiles = nchunks * bpc;
  const unsigned g = (unsigned)bounded_grid(sh, cus, ntiles), b = (unsigned)bpc;
  return with_policy(sh, [&](auto ntl, auto sp) {
    return launch_k(k_reduce_bounded<P, NOUT, V, decltype(ntl)::value, decltype(sp)::value>, g, dim3(sh.block), 0,
                    st, in, out, e0, e1, chunk, b, ntiles);
  });
}

template <int P, int NOUT>
hipError_t bounded_p(const Shape& sh, int cus, hipStream_t st, const InPtrs& in, const OutPtrs& out, size_t e0,
                     size_t e1, size_t chunk) {
  if (sh.vec == 2) return bounded_v<P, NOUT, 2>(sh, cus, st, in, out, e0, e1, chunk);
  return bounded_v<P, NOUT, 1>(sh, cus, st, in, out, e0, e1, chunk);
}

template <int P, int NOUT>
hipError_t range_p(const Shape& sh, hipStream_t st, const InPtrs& in, const OutPtrs& out, size_t e0,
                   size_t e1, size_t chunk, const ChunkSignal& sig = ChunkSignal{nullptr, nullptr, 0, 0}) {
  if (sh.vec == 2) return range_v<P, NOUT, 2>(sh, st, in, out, e0, e1, chunk, sig);
  return range_v<P, NOUT, 1>(sh, st, in, out, e0, e1, chunk, sig);
}

template <int P, int BLOCK>
hipError_t oneshot_small_b(const Shape& sh, hipStream_t st, const InPtrs& in, void* out, size_t n) {
  const size_t blocks = cdiv(n, (size_t)BLOCK * 8);
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
  return with_policy(sh, [&](auto ntl, auto sp) {
    return launch_k(k_oneshot_small<P, BLOCK, decltype(ntl)::value, decltype(sp)::value>, (unsigned)blocks,
                    dim3(BLOCK), sh.lds, st, in, out, n);
  });
}

// The compact kernel for one group per lane; a shape with two groups per
// lane takes k_reduce.
template <int P>
hipError_t oneshot_small_p(const Shape& sh, hipStream_t st, const InPtrs& in, void* out, size_t n) {
  if (sh.vec == 1) {
    if (sh.block == 64) return oneshot_small_b<P, 64>(sh, st, in, out, n);
    if (sh.block == 128) return oneshot_small_b<P, 128>(sh, st, in, out, n);
    if (sh.block == 256) return oneshot_small_b<P, 256>(sh, st, in, out, n);
  }
  OutPtrs o{};
  o.p[0] = out;
  return range_p<P, 1>(sh, st, in, o, 0, n, n);
}

template <int P, int BLOCK>
hipError_t inplace_small_b(const Shape& sh, hipStream_t st, const OutPtrs& io, size_t n) {
  const size_t blocks = cdiv(n, (size_t)BLOCK * 8);
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
  return with_policy(sh, [&](auto ntl, auto sp) {
    return launch_k(k_2stage_small_inplace<P, BLOCK, decltype(ntl)::value, decltype(sp)::value>, (unsigned)blocks,
                    dim3(BLOCK), sh.lds, st, io, n);
  });
}

template <int P, int BLOCK>
hipError_t offs_small_b(const Shape& sh, hipStream_t st, const PtrOffsets& po, size_t n) {
  const size_t blocks = cdiv(n, (size_t)BLOCK * 8);
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
  return with_policy(sh, [&](auto ntl, auto sp) {
    return launch_k(k_2stage_small_offs<P, BLOCK, decltype(ntl)::value, decltype(sp)::value>, (unsigned)blocks,
                    dim3(BLOCK), sh.lds, st, po, n);
  });
}

// Fused two-stage for small messages, with one group per lane: in place
// (every output its own input) the in-place kind's shape and its compact
// kernel; with separate outputs the small kind's shape and, when every
// buffer's offset from ins[0] fits pack_offsets, the offset-argument kernel.
// Otherwise k_reduce.
template <int P>
hipError_t fused_small_p(const Launch& L, const InPtrs& in, const OutPtrs& out, size_t n) {
  bool inplace = true;
  for (int p = 0; p < P; ++p) inplace = inplace && out.p[p] == in.p[p];
  const Shape& sh = inplace ? L.shape[k2StageInplaceSmall] : L.shape[k2StageSmall];
  if (inplace && sh.vec == 1) {
    if (sh.block == 64) return inplace_small_b<P, 64>(sh, L.stream, out, n);
    if (sh.block == 128) return inplace_small_b<P, 128>(sh, L.stream, out, n);
    if (sh.block == 256) return inplace_small_b<P, 256>(sh, L.stream, out, n);
  }
  PtrOffsets po;
  const void* ptrs[2 * AR_MAX_RANKS];
  for (int p = 0; p < P; ++p) {
    ptrs[p] = in.p[p];
    ptrs[P + p] = out.p[p];
  }
  if (!inplace && sh.vec == 1 && pack_offsets(ptrs, 2 * P, &po)) {
    if (sh.block == 64) return offs_small_b<P, 64>(sh, L.stream, po, n);
    if (sh.block == 128) return offs_small_b<P, 128>(sh, L.stream, po, n);
    if (sh.block == 256) return offs_small_b<P, 256>(sh, L.stream, po, n);
  }
  return range_p<P, P>(sh, L.stream, in, out, 0, n, n);
}

template <int P>
hipError_t staged_p(const Launch& L, const InPtrs& in, const OutPtrs& out, size_t n, void* scratch) {
  const size_t S = cdiv(cdiv(n, 8), P) * 8;
  const Shape& rs = L.shape[kRS];
  const Shape& ag = L.shape[kAG];
  const size_t bps_rs = cdiv(S / 8, (size_t)rs.block), bps_ag = cdiv(S / 8, (size_t)ag.block);
  // both grids are checked before the first launch
  if (bps_rs * P > 0x7FFFFFFFull || bps_ag * P > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
  const unsigned g_rs = (unsigned)(bps_rs * P), g_ag = (unsigned)(bps_ag * P);
  auto rs_go = [&](auto blk) {
    return with_policy(rs, [&](auto ntl, auto sp) {
      return launch_k(k_rs<P, decltype(blk)::value, decltype(ntl)::value, decltype(sp)::value>, g_rs,
                      dim3(decltype(blk)::value), rs.lds, L.stream, in, scratch, n, S);
    });
  };
  auto ag_go = [&](auto blk) {
    return with_policy(ag, [&](auto ntl, auto sp) {
      return launch_k(k_ag<P, decltype(blk)::value, decltype(ntl)::value, decltype(sp)::value>, g_ag,
                      dim3(decltype(blk)::value), ag.lds, L.stream, (const void*)scratch, out, n, S);
    });
  };
  // the shape table holds only 64-, 128- or 256-lane blocks for these kinds
  hipError_t e = rs.block == 64 ? rs_go(SPc<64>{}) : rs.block == 128 ? rs_go(SPc<128>{}) : rs_go(SPc<256>{});
  if (e != hipSuccess) return e;
  return ag.block == 64 ? ag_go(SPc<64>{}) : ag.block == 128 ? ag_go(SPc<128>{}) : ag_go(SPc<256>{});
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
  if (n <= (size_t)AR_SMALL_ELEMS) {
    AR_DISPATCH_P(P, (oneshot_small_p<PP>(L.shape[kOneshotSmall], L.stream, in, out, n)))
  }
  OutPtrs o{};
  o.p[0] = out;
  AR_DISPATCH_P(P, (range_p<PP, 1>(L.shape[kOneshot], L.stream, in, o, 0, n, n)))
}

hipError_t launch_2stage_fused(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                               size_t n) {
  if (n <= (size_t)AR_SMALL_ELEMS) {
    AR_DISPATCH_P(P, (fused_small_p<PP>(L, in, out, n)))
  }
  AR_DISPATCH_P(P, (range_p<PP, PP>(L.shape[k2Stage], L.stream, in, out, 0, n, n)))
}

hipError_t launch_2stage_staged(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                                size_t n, void* scratch) {
  AR_DISPATCH_P(P, (staged_p<PP>(L, in, out, n, scratch)))
}

// The grid check of range_v / bounded_v, without launching.
bool chunked_fits(const Launch& L, size_t e0, size_t e1, size_t chunk_elems, int two_stage, bool flags,
                  bool bounded) {
  const Shape& sh = bounded ? L.shape[kUbatchBounded]
                            : (flags ? L.shape[kUbatchFlags] : (two_stage ? L.shape[kUbatch] : L.shape[kOneshot]));
  const size_t span = (size_t)(sh.vec == 2 ? 2 : 1) * sh.block * 8;
  const size_t bpc = cdiv(chunk_elems, span);
  const size_t nchunks = cdiv(e1 - e0, chunk_elems);
  if (bounded) return bpc <= 0xFFFFFFFFull && nchunks <= (~(size_t)0) / bpc;
  return bpc <= 0x7FFFFFFFull && nchunks <= 0x7FFFFFFFull / bpc;
}

hipError_t launch_chunked_bounded(const Launch& L, const InPtrs& in, const OutPtrs& out, int P, size_t e0,
                                  size_t e1, size_t chunk_elems, int two_stage) {
  const Shape& sh = L.shape[kUbatchBounded];
  if (two_stage) {
    AR_DISPATCH_P(P, (bounded_p<PP, PP>(sh, L.cus, L.stream, in, out, e0, e1, chunk_elems)))
  }
  AR_DISPATCH_P(P, (bounded_p<PP, 1>(sh, L.cus, L.stream, in, out, e0, e1, chunk_elems)))
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
