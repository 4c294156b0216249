// fp8-quantised contributions ("[DSV4] perf(tbo): overlap pure-TP all_reduce
// on TBO + Delay TP", reviewed diff: the custom all-reduce call site passes a
// ca_fp8_quant flag; the page gives no scheme).  The reading implemented:
// each rank's bf16 buffer travels as E4M3 codes (OCP "FN": bias 7, no
// infinities, 0x7F / 0xFF are NaN, largest finite 448) with one
// power-of-two scale byte per block of 32 consecutive elements; the scale is
// the smallest power of two at which no element of the block exceeds 448,
// so nothing clips.  The receiver dequantises exactly (code value times the
// scale) and sums in binary32 in rank order 0..P-1, then rounds once to bf16.
//
// Quantise: one lane per 8 elements (16 bytes of bf16 in, 8 code bytes out);
// the 4 lanes of a quad hold one 32-element block and find its largest
// magnitude with two DPP lane swaps.  x / 2^k is exact (a power-of-two
// scaling), so the hardware E4M3 conversion (round to nearest even) gives
// the code of the exact quotient.
// Reduce: one lane per 8 or 16 elements (one 8- or 16-byte load of codes per
// rank plus its block's scale byte), hardware E4M3 -> binary32 conversion (exact),
// ldexp by the scale (exact), rank-order binary32 sums, the integer
// nearest-even rounding to bf16 shared with the other reduce kernels.
#include "ar_device.hpp"
#include "ar_internal.hpp"

namespace ar {
namespace {

constexpr int kFp8Block = 32;

// Largest of the 4 values held by one quad of lanes (lanes 4q..4q+3).
// DPP quad permutations [1,0,3,2] and [2,3,0,1]; every lane must be active.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  return v;
}

// Scale exponent k from the binary32 bits A of the block's largest finite
// magnitude: the smallest k in [-127, 127] with A <= 448 * 2^k.  For a
// normal A = (1 + F/2^23) * 2^(E-127) and 448 = 1.75 * 2^8, that is E - 135,
// plus one when the significand exceeds 1.75 (F > 0x600000).  Zero and
// binary32 subnormals (below 2^-126, far below 448 * 2^-127) give -127;
// the largest finite bf16 gives 120, so no upper clamp is reached.
__device__ __forceinline__ int fp8_scale_exp(uint32_t A) {
  const int E = (int)(A >> 23);
  if (E == 0) return -127;
  const int k = E - 135 + ((A & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return k < -127 ? -127 : k;
}

// Binary32 bits of bf16 element j (0..7) of a 16-byte group.
__device__ __forceinline__ uint32_t elem_bits(const uint32_t (&w)[4], int j) {
  return (j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16);
}

// Codes of 4 elements (bits b[0..3]) scaled by 2^-k, as one little-endian
// word; a NaN or infinite element gives 0x7F.
__device__ __forceinline__ uint32_t codes4(const uint32_t* b, int k) {
  const float s0 = __builtin_ldexpf(__uint_as_float(b[0]), -k);
  const float s1 = __builtin_ldexpf(__uint_as_float(b[1]), -k);
  const float s2 = __builtin_ldexpf(__uint_as_float(b[2]), -k);
  const float s3 = __builtin_ldexpf(__uint_as_float(b[3]), -k);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(s0, s1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(s2, s3, w, true);
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if ((b[j] & 0x7FFFFFFFu) >= 0x7F800000u) bad |= 0xFFu << (8 * j);
  return ((uint32_t)w & ~bad) | (0x7F7F7F7Fu & bad);
}

// Workgroup b quantises tile b % tiles of buffer b / tiles; a tile is
// V * blockDim groups of 8 elements.  Lanes past the end take part in the
// quad maximum with zeros and store nothing.
template <int V, bool NTL, int SP>
__global__ __launch_bounds__(kMaxBlock) void k_quant_fp8(InPtrs xs, ByteOut codes, ByteOut scales,
                                                         size_t n, unsigned tiles) {
  const unsigned p = blockIdx.x / tiles;
  const size_t tile0 = (size_t)(blockIdx.x % tiles) * V * blockDim.x;
  const u32x4* x4 = static_cast<const u32x4*>(xs.p[p]);
  const uint16_t* x16 = static_cast<const uint16_t*>(xs.p[p]);
  uint8_t* cp = codes.p[p];
  uint8_t* sp = scales.p[p];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t g = tile0 + (size_t)u * blockDim.x + threadIdx.x;
    const size_t i0 = g * 8;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (i0 + 8 <= n) {
      const u32x4 v = ld4<NTL>(x4 + g);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t e = i0 + j < n ? (uint32_t)x16[i0 + j] : 0u;
        w[j >> 1] |= (j & 1) ? (e << 16) : e;
      }
    }
    uint32_t b[8];
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      b[j] = elem_bits(w, j);
      const uint32_t a = b[j] & 0x7FFFFFFFu;
      if (a < 0x7F800000u) amax = max(amax, a);
    }
    amax = quad_max(amax);
    const int k = fp8_scale_exp(amax);
    const uint32_t lo = codes4(b, k), hi = codes4(b + 4, k);
    if (i0 + 8 <= n) {
      const uint64_t c = (uint64_t)lo | ((uint64_t)hi << 32);
      st8p<SP>(reinterpret_cast<uint64_t*>(cp) + tile0 + (size_t)u * blockDim.x, blockDim.x * 8u, threadIdx.x * 8u, c);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (i0 + j < n) cp[i0 + j] = (uint8_t)(((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xFFu);
    }
    if ((threadIdx.x & 3u) == 0 && i0 < n) sp[g >> 2] = (uint8_t)(k + 127);
  }
}

// Binary32 value of codes byte-pairs: element 2h and 2h+1 of word w.
__device__ __forceinline__ void dequant4(uint32_t w, int k, float* d) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  d[0] = __builtin_ldexpf(lo[0], k);
  d[1] = __builtin_ldexpf(lo[1], k);
  d[2] = __builtin_ldexpf(hi[0], k);
  d[3] = __builtin_ldexpf(hi[1], k);
}

// Lane g reduces elements [EPL*g, EPL*g + EPL): EPL / 4 code words of every
// rank (one 8- or 16-byte load) and the scale byte of their block, and
// stores EPL / 8 16-byte groups to every output.  EPL = 8 (one 16-byte store
// per output) measured about 10% faster than 16 for the 8-output reduce.  A
// group that runs past n is done element by element by its lane.
template <int EPL, bool NT>
__device__ __forceinline__ void load_codes(const uint8_t* c, size_t g, uint32_t (&w)[EPL / 4]) {
  if constexpr (EPL == 8) {
    const uint64_t* p = reinterpret_cast<const uint64_t*>(c) + g;
    uint64_t v;
    if constexpr (NT) v = __builtin_nontemporal_load(p);
    else v = *p;
    w[0] = (uint32_t)v;
    w[1] = (uint32_t)(v >> 32);
  } else {
    const u32x4 v = ld4<NT>(reinterpret_cast<const u32x4*>(c) + g);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
}

template <int P, int NOUT, int EPL, bool NTL, int SP>
__global__ __launch_bounds__(kMaxBlock) void k_reduce_fp8(ByteIn codes, ByteIn scales, OutPtrs out,
                                                          size_t n) {
  constexpr int NW = EPL / 4;
  // Workgroups reach the 8 XCDs round-robin.  A 128-byte line of scale bytes
  // covers G = 4096 / (blockDim.x * EPL) consecutive tiles (8 at 64 lanes x
  // 8 elements, 4 at 128 lanes, 2 at 256).  Within every run of 8 G
  // workgroups, XCD x takes the G consecutive tiles x G .. x G + G - 1, so
  // the tiles that share a scale line meet in one XCD's L2 instead of
  // fetching it once per XCD.  The last, partial run keeps the identity
  // order; every tile is still taken exactly once.
  const unsigned G = 4096u / (blockDim.x * (unsigned)EPL);
  size_t tile = blockIdx.x;
  if (G > 1) {
    const size_t R = 8 * (size_t)G;
    if ((size_t)(blockIdx.x / R + 1) * R <= gridDim.x)
      tile = (size_t)(blockIdx.x / R) * R + (blockIdx.x % 8) * G + (blockIdx.x / 8) % G;
  }
  const size_t g = tile * blockDim.x + threadIdx.x;
  const size_t i0 = g * EPL;
  if (i0 >= n) return;
  if (i0 + EPL <= n) {
    uint32_t cw[P][NW];
    int k[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      load_codes<EPL, NTL>(codes.p[p], g, cw[p]);
      k[p] = (int)scales.p[p][i0 / kFp8Block] - 127;
    }
    float acc[EPL];
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        float d[4];
        dequant4(cw[p][q], k[p], d);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * q + j] = p == 0 ? d[j] : acc[4 * q + j] + d[j];
      }
    }
#pragma unroll
    for (int h = 0; h < EPL / 8; ++h) {
      u32x4 r;
      r.x = pack_bf16x2(acc[8 * h + 0], acc[8 * h + 1]);
      r.y = pack_bf16x2(acc[8 * h + 2], acc[8 * h + 3]);
      r.z = pack_bf16x2(acc[8 * h + 4], acc[8 * h + 5]);
      r.w = pack_bf16x2(acc[8 * h + 6], acc[8 * h + 7]);
#pragma unroll
      for (int o = 0; o < NOUT; ++o)
        st16<SP>(static_cast<u32x4*>(out.p[o]) + (EPL / 8) * tile * blockDim.x, (EPL / 8) * blockDim.x * 16u,
                 ((EPL / 8) * threadIdx.x + h) * 16u, r);
    }
  } else {
    for (size_t i = i0; i < n; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const float v = __builtin_amdgcn_cvt_f32_fp8((int)codes.p[p][i], 0);
        const float d = __builtin_ldexpf(v, (int)scales.p[p][i / kFp8Block] - 127);
        acc = p == 0 ? d : acc + d;
      }
      const uint16_t r = (uint16_t)(rne_hi(acc) >> 16);
#pragma unroll
      for (int o = 0; o < NOUT; ++o) static_cast<uint16_t*>(out.p[o])[i] = r;
    }
  }
}

template <int V>
hipError_t quant_v(const Shape& sh, hipStream_t st, const InPtrs& xs, const ByteOut& codes,
                   const ByteOut& scales, int P, size_t n) {
  const size_t groups = cdiv(n, 8);
  const size_t tiles = cdiv(groups, (size_t)V * sh.block);
  if (tiles * (size_t)P > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
  const unsigned g = (unsigned)(tiles * P), t = (unsigned)tiles;
  const dim3 blk(sh.block);
  return with_policy(sh, [&](auto ntl, auto sp) {
    return launch_k(k_quant_fp8<V, decltype(ntl)::value, decltype(sp)::value>, g, blk, sh.lds, st, xs, codes, scales,
                    n, t);
  });
}

template <int P, int NOUT, int EPL>
hipError_t reduce_e(const Shape& sh, hipStream_t st, const ByteIn& codes, const ByteIn& scales,
                    const OutPtrs& out, size_t n) {
  const size_t blocks = cdiv(cdiv(n, (size_t)EPL), (size_t)sh.block);
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
  const unsigned g = (unsigned)blocks;
  const dim3 blk(sh.block);
  return with_policy(sh, [&](auto ntl, auto sp) {
    return launch_k(k_reduce_fp8<P, NOUT, EPL, decltype(ntl)::value, decltype(sp)::value>, g, blk, sh.lds, st, codes,
                    scales, out, n);
  });
}

// The shape's vec counts 16-byte output groups per lane: 1 -> 8 elements,
// 2 -> 16 elements per lane.
template <int P>
hipError_t reduce_p(const Shape& sh, hipStream_t st, const ByteIn& codes, const ByteIn& scales,
                    const OutPtrs& out, int nout, size_t n) {
  if (nout == 1) {
    if (sh.vec == 2) return reduce_e<P, 1, 16>(sh, st, codes, scales, out, n);
    return reduce_e<P, 1, 8>(sh, st, codes, scales, out, n);
  }
  if (sh.vec == 2) return reduce_e<P, P, 16>(sh, st, codes, scales, out, n);
  return reduce_e<P, P, 8>(sh, st, codes, scales, out, n);
}

}  // namespace

hipError_t launch_quant_fp8(const Launch& L, const InPtrs& xs, const ByteOut& codes,
                            const ByteOut& scales, int P, size_t n) {
  const Shape& sh = L.shape[kQuantFp8];
  if (sh.vec == 2) return quant_v<2>(sh, L.stream, xs, codes, scales, P, n);
  return quant_v<1>(sh, L.stream, xs, codes, scales, P, n);
}

hipError_t launch_reduce_fp8(const Launch& L, const ByteIn& codes, const ByteIn& scales,
                             const OutPtrs& out, int P, int nout, size_t n) {
  const Shape& sh = L.shape[nout == 1 ? kReduceFp8 : kReduceFp8All];
  switch (P) {
    case 1: return reduce_p<1>(sh, L.stream, codes, scales, out, nout, n);
    case 2: return reduce_p<2>(sh, L.stream, codes, scales, out, nout, n);
    case 3: return reduce_p<3>(sh, L.stream, codes, scales, out, nout, n);
    case 4: return reduce_p<4>(sh, L.stream, codes, scales, out, nout, n);
    case 5: return reduce_p<5>(sh, L.stream, codes, scales, out, nout, n);
    case 6: return reduce_p<6>(sh, L.stream, codes, scales, out, nout, n);
    case 7: return reduce_p<7>(sh, L.stream, codes, scales, out, nout, n);
    case 8: return reduce_p<8>(sh, L.stream, codes, scales, out, nout, n);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ar
