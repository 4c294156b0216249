// Buffer offsets for the compact small-message fused two-stage kernel.
//
// HIP enqueues a kernel about 0.7 us faster when its whole argument segment
// is at most 112 bytes; 2P buffer pointers and n are 136 bytes at P = 8.  The
// kernel therefore takes one base pointer (ins[0]) and the other 2P - 1
// buffers as signed 32-bit offsets from it, in units of 2^shift bytes, where
// 2^shift is the largest power of two, at most 2^30, that divides every
// difference.  With the 16-byte alignment every data pointer has, shift >= 4
// and the reach is at least +-32 GiB; with 512-byte aligned allocations it
// is +-1 TiB.  The struct is 72 bytes (shift sits in what would be padding),
// 80 with n.
//
// Plain C++ with no HIP dependency, so the host-side arithmetic can be
// compiled and checked on its own.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ar.h"

namespace ar {

struct PtrOffsets {
  const char* base;                   // ins[0]
  int32_t off[2 * AR_MAX_RANKS - 1];  // ins[1..P-1], then outs[0..P-1], in units of 2^shift bytes
  uint32_t shift;
};

// ptrs[0..count-1]: ins[0..P-1] then outs[0..P-1] (count = 2P, at most
// 2 * AR_MAX_RANKS).  Fills *po and returns true when every offset from
// ptrs[0] fits; returns false (and *po is unspecified) otherwise.
inline bool pack_offsets(const void* const* ptrs, int count, PtrOffsets* po) {
  if (count < 1 || count > 2 * AR_MAX_RANKS) return false;
  const uintptr_t b = reinterpret_cast<uintptr_t>(ptrs[0]);
  int64_t d[2 * AR_MAX_RANKS - 1] = {};
  uintptr_t bits = 0;
  for (int i = 1; i < count; ++i) {
    // modular difference, read as signed: exact for two addresses of one
    // device, which lie far less than 2^63 bytes apart
    const uintptr_t u = reinterpret_cast<uintptr_t>(ptrs[i]) - b;
    d[i - 1] = static_cast<int64_t>(u);
    bits |= u;
  }
  unsigned shift = 0;
  while (shift < 30 && ((bits >> shift) & 1u) == 0) ++shift;
  po->base = static_cast<const char*>(ptrs[0]);
  po->shift = shift;
  for (int i = 0; i < 2 * AR_MAX_RANKS - 1; ++i) {
    const int64_t q = d[i] / (static_cast<int64_t>(1) << shift);  // exact: 2^shift divides every difference
    if (q < INT32_MIN || q > INT32_MAX) return false;
    po->off[i] = static_cast<int32_t>(q);
  }
  return true;
}

// The address the kernel rebuilds from an offset (constexpr, so HIP
// compiles it for the device too).
constexpr const char* offset_address(const PtrOffsets& po, int i) {
  return po.base + static_cast<int64_t>(po.off[i]) * (static_cast<int64_t>(1) << po.shift);
}

}  // namespace ar
