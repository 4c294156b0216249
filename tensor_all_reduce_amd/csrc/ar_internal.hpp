// Internal interface between the C-ABI layer (ar_api.hip) and the kernel
// translation units (ar_reduce.hip, ar_fused.hip).  Not installed; the public
// boundary is include/ar.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "ar.h"

namespace ar {

// Per-kernel launch shape.  Every streaming kernel runs on a flat grid of
// `block`-lane workgroups, each owning a contiguous tile of vec * block
// 16-byte groups.  `wg_per_cu` caps how many workgroups share a CU by
// requesting lds = (LDS per CU) / wg_per_cu bytes of dynamic LDS that the
// kernel never touches: fewer waves in flight means fewer reads and writes
// interleaved at the memory controller, which measured up to 13% faster for
// the 8 -> 8 patterns.
struct Shape {
  int block;      // 64, 128 or 256 lanes
  int vec;        // 1 or 2: work per lane (16-byte groups per buffer for the
                  // reduces; the lane width for pack, unpack and the fp8 reduce)
  int nt_loads;   // 1: non-temporal loads of streamed inputs
  int stores;     // output store policy: 0 plain, 1 NT, 2 SC1, 3 SC1 + NT (st16)
  int wg_per_cu;  // 0: no cap
  unsigned lds;   // resolved dynamic LDS bytes per workgroup
};

enum Kind {
  kOneshot = 0,  // 8 -> 1 reduce
  k2Stage,       // 8 -> 8 fused reduce (write mode)
  kUbatch,       // 8 -> 8 chunked reduce, two concurrent streams
  kRS,           // staged reduce-scatter: 8 -> scratch
  kAG,           // staged all-gather: scratch -> 8
  kPack,         // 1 -> 2 (bf16 -> payload words)
  kUnpack,       // 2 -> 1 (payload words -> bf16)
  kRD,           // fused recursive doubling, 8 payloads -> 8 payloads
  kRDStep,       // staged recursive-doubling step
  kUnpackWait,   // unpack that waits for the producer (persistent grid, no LDS request)
  kUbatchFlags,  // chunked reduce that publishes per-chunk completion flags
  kQuantFp8,     // bf16 -> fp8 codes + block scales, P buffers in one launch
  kReduceFp8,    // P fp8 contributions -> 1 bf16 output
  kReduceFp8All, // P fp8 contributions -> P bf16 outputs
  kOneshotSmall, // kOneshot for n <= AR_SMALL_ELEMS
  k2StageSmall,  // k2Stage for n <= AR_SMALL_ELEMS
  kRDSmall,      // kRD for n <= AR_SMALL_ELEMS
  kRDStepSmall,  // kRDStep for n <= AR_SMALL_ELEMS
  kPackSmall,    // kPack for n <= AR_SMALL_ELEMS
  kUnpackSmall,  // kUnpack for n <= AR_SMALL_ELEMS
  kUbatchBounded, // chunked reduce on a persistent grid of a fraction of the CUs
  k2StageInplaceSmall, // k2StageSmall when every output is its own input
  kKinds
};

// Launch policy for one call, resolved by the API layer from the per-device
// cache and the shape table (read once).
struct Launch {
  int cus;             // compute units on the current device
  const Shape* shape;  // kKinds resolved shapes (an immutable per-device table)
  void* scratch;       // this device's static scratch array (ar_reduce_2stage_static)
  hipStream_t stream;
};

// The shape of a whole-buffer call over n elements per rank: a message of at
// most AR_SMALL_ELEMS elements takes its small-message kind.
inline const Shape& shape_for(const Launch& L, Kind large, Kind small, size_t n) {
  return n <= (size_t)AR_SMALL_ELEMS ? L.shape[small] : L.shape[large];
}

// Calls f(NTL, SP) with the shape's load hint and store policy as
// compile-time constants (std::integral_constant), so a launcher picks the
// kernel instantiation in one place.
template <int S> using SPc = std::integral_constant<int, S>;
template <typename F>
inline hipError_t with_policy(bool nt_loads, int stores, F&& f) {
  if (nt_loads) {
    switch (stores) {
      case 0: return f(std::true_type{}, SPc<0>{});
      case 1: return f(std::true_type{}, SPc<1>{});
      case 2: return f(std::true_type{}, SPc<2>{});
      default: return f(std::true_type{}, SPc<3>{});
    }
  }
  switch (stores) {
    case 0: return f(std::false_type{}, SPc<0>{});
    case 1: return f(std::false_type{}, SPc<1>{});
    case 2: return f(std::false_type{}, SPc<2>{});
    default: return f(std::false_type{}, SPc<3>{});
  }
}
template <typename F>
inline hipError_t with_policy(const Shape& sh, F&& f) {
  return with_policy(sh.nt_loads != 0, sh.stores, static_cast<F&&>(f));
}

// Pointer bundles passed to kernels by value (kernel arguments), so no
// device-side pointer table and no host->device copy is needed per call.
struct InPtrs { const void* p[AR_MAX_RANKS]; };
struct OutPtrs { void* p[AR_MAX_RANKS]; };
struct WordIn { const uint64_t* p[AR_MAX_RANKS]; };
// Per-chunk completion signal of the chunked reduce (done == nullptr: none).
struct ChunkSignal {
  uint32_t* done;    // done[base + c] = epoch once chunk c is fully written
  uint32_t* tiles;   // per-chunk tile counters, zero between calls
  uint32_t epoch;
  uint32_t base;     // index of this launch's first chunk in done / tiles
};
struct WordOut { uint64_t* p[AR_MAX_RANKS]; };
struct ByteIn { const uint8_t* p[AR_MAX_RANKS]; };
struct ByteOut { uint8_t* p[AR_MAX_RANKS]; };

hipError_t launch_oneshot(const Launch& L, const InPtrs& in, int P, void* out, size_t n);
hipError_t launch_2stage_fused(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                               size_t n);
hipError_t launch_2stage_staged(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                                size_t n, void* scratch);
// Chunked reduce of elements [e0, e1) of every buffer, chunk-major workgroups.
hipError_t launch_chunked(const Launch& L, const InPtrs& in, const OutPtrs& out, int P,
                          size_t e0, size_t e1, size_t chunk_elems, int two_stage,
                          const ChunkSignal& sig);
// Chunked reduce of [e0, e1) on the bounded persistent grid (kUbatchBounded).
hipError_t launch_chunked_bounded(const Launch& L, const InPtrs& in, const OutPtrs& out, int P, size_t e0,
                                  size_t e1, size_t chunk_elems, int two_stage);
// Whether the grid of launch_chunked (or launch_chunked_bounded) for
// [e0, e1) fits a launch (checked by the API layer before any launch of a
// multi-launch call).
bool chunked_fits(const Launch& L, size_t e0, size_t e1, size_t chunk_elems, int two_stage, bool flags,
                  bool bounded);

hipError_t launch_quant_fp8(const Launch& L, const InPtrs& xs, const ByteOut& codes,
                            const ByteOut& scales, int P, size_t n);
hipError_t launch_reduce_fp8(const Launch& L, const ByteIn& codes, const ByteIn& scales,
                             const OutPtrs& out, int P, int nout, size_t n);

hipError_t launch_pack(const Launch& L, const void* x, uint64_t* w, size_t n, uint32_t seq);
hipError_t launch_unpack(const Launch& L, const uint64_t* w, void* x, size_t n, uint32_t seq,
                         uint64_t* d_err);
hipError_t launch_rd_fused(const Launch& L, const WordIn& in, const WordOut& out, int P,
                           size_t n, uint32_t seq0, int fp32_carry, uint64_t* d_err);
hipError_t launch_rd_staged(const Launch& L, const WordIn& in, const WordOut& out, int P,
                            size_t n, uint32_t seq0, uint64_t* mailbox, uint64_t* d_err);
hipError_t launch_unpack_wait(const Launch& L, const uint64_t* w, void* x, size_t n, uint32_t seq,
                              uint32_t max_spins, uint64_t* d_err);
hipError_t launch_err_init(const Launch& L, uint64_t* d_err);

}  // namespace ar
