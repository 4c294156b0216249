// Device-side building blocks shared by the gfx950 kernels.
//
// Data movement: every streamed access is a 128-bit (dwordx4) vector access,
// one per lane, so a 64-lane wavefront touches 1 KiB of contiguous memory per
// instruction.  bf16 values are carried as raw 16-bit halves of 32-bit words:
// element 2k of a 16-byte group is the low half of word k, element 2k+1 the
// high half.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace ar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxBlock = 256;  // largest workgroup the kernels are compiled for
constexpr int kMaxBlockBounded = 1024;  // ... except the bounded-footprint reduce
constexpr int kWave = 64;       // CDNA wavefront width

template <bool NT>
__device__ __forceinline__ u32x4 ld4(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__device__ __forceinline__ void st4(u32x4* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <bool NT>
__device__ __forceinline__ uint64_t ld8(const uint64_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__device__ __forceinline__ void st8(uint64_t* p, uint64_t v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Output store policy, the launch shape's `stores` field:
//   0  plain store (write-back through the XCD's L2);
//   1  non-temporal (streaming hint);
//   2  SC1: written through past the XCD's L2 to the level every XCD sees;
//   3  SC1 + non-temporal.
// Policies 2 and 3 are buffer stores carrying the cache-policy bits (aux bit
// 4 = SC1, bit 1 = NT).  They measured faster than the plain and
// non-temporal forms for every streamed output on MI355X (e.g. the fused
// 8 -> 8 reduce at 256 MiB per buffer 684.6 -> 674.2 us, the 8 -> 1 one-shot
// 380 -> 366 us), and they are what makes data covered by a completion flag
// visible to another XCD without an L2 writeback: once the wave's store
// counter drains, no dirty copy sits in one XCD's L2.
//
// Every helper takes the wave-uniform start of the written span (`base`),
// its length in bytes (the buffer descriptor's range) and this lane's byte
// offset in it; policies 0 and 1 simply store to base + off.  Descriptor
// word 3 = 0x00020000 selects the 32-bit data format (any nonzero format
// works for untyped access).
template <int SP>
__device__ __forceinline__ void st16(void* base, uint32_t bytes, uint32_t off, u32x4 v) {
  if constexpr (SP >= 2) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, SP == 3 ? (16 | 2) : 16);
  } else {
    st4<SP == 1>(reinterpret_cast<u32x4*>(static_cast<char*>(base) + off), v);
  }
}

template <int SP>
__device__ __forceinline__ void st8p(void* base, uint32_t bytes, uint32_t off, uint64_t v) {
  if constexpr (SP >= 2) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
    const u32x2 w = {(uint32_t)v, (uint32_t)(v >> 32)};
    __builtin_amdgcn_raw_buffer_store_b64(w, rs, (int)off, 0, SP == 3 ? (16 | 2) : 16);
  } else {
    st8<SP == 1>(reinterpret_cast<uint64_t*>(static_cast<char*>(base) + off), v);
  }
}

// s_waitcnt with vmcnt = 0 and expcnt / lgkmcnt left at their maxima (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8): the wave
// waits until all of its vector memory operations, stores included, are
// acknowledged.
constexpr int kWaitVmcnt0 = 0x0F70;

// bf16 -> binary32 is exact: the bf16 bits are the high half of the float.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// binary32 -> bf16, round to nearest, ties to even, returned in the HIGH half
// of the word (low half is don't-care).  Adding 0x7FFF plus the lowest kept
// bit carries into the kept half exactly when the discarded half is above
// one half, or equal to one half with an odd kept half.  A NaN (whose
// payload the addition could carry into the exponent) is replaced by the
// canonical quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t rne_hi(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
  return __builtin_isnan(f) ? 0x7FC00000u : r;
}

// Round and re-widen: the binary32 value of rne(f).
__device__ __forceinline__ float round_bf16(float f) {
  return __uint_as_float(rne_hi(f) & 0xFFFF0000u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (rne_hi(lo) >> 16) | (rne_hi(hi) & 0xFFFF0000u);
}

__device__ __forceinline__ uint16_t to_bf16(float f) { return (uint16_t)(rne_hi(f) >> 16); }

// Sum of P 16-byte groups (8 bf16 each) in rank order 0..P-1, binary32
// accumulation starting from rank 0, one rounding per element.
template <int P>
__device__ __forceinline__ u32x4 reduce8(const u32x4 (&x)[P]) {
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float lo = lo_f32(x[0][k]);
    float hi = hi_f32(x[0][k]);
#pragma unroll
    for (int p = 1; p < P; ++p) {
      lo = lo + lo_f32(x[p][k]);
      hi = hi + hi_f32(x[p][k]);
    }
    o[k] = pack_bf16x2(lo, hi);
  }
  return o;
}

template <int P>
__device__ __forceinline__ uint16_t reduce1(const uint16_t* const* in16, size_t i) {
  float acc = bf16_f32(in16[0][i]);
#pragma unroll
  for (int p = 1; p < P; ++p) acc = acc + bf16_f32(in16[p][i]);
  return to_bf16(acc);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Launch through hipLaunchKernel so the launch status is returned directly
// instead of being read back from the thread's sticky last-error slot.
template <typename T> struct id { using type = T; };

// `lds` bytes of dynamic LDS per workgroup are requested only to cap how many
// workgroups share a CU (an occupancy knob); no kernel reads them.
template <typename... KArgs>
inline hipError_t launch_k(void (*k)(KArgs...), dim3 grid, dim3 block, unsigned lds, hipStream_t s,
                           typename id<KArgs>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, lds, s);
}

inline size_t cdiv(size_t a, size_t b) { return (a + b - 1) / b; }

}  // namespace ar
