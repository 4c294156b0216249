// Fused-payload kernels for gfx950: pack, unpack with sequence-number
// validation, and the recursive-doubling combine (fused and staged).
//
// Page cited: [NVRAR] "Technical Summary: Understanding and Improving
// Communication Performance in Multi-node LLM Inference", Methodology 3
// (phase 2, "Inter-node Recursive-Doubling") and Optimizations ("Fused
// Payloads": data and flag in one 8-byte word; "Sequence-Number
// Synchronization": a unique sequence number marks a payload as current).
//
// Payload word j (little-endian u64): low 32 bits = the 32-bit word holding
// bf16 elements 2j (low half) and 2j+1 (high half); high 32 bits = sequence
// number.  In memory a 16-byte group of payload is therefore the u32 stream
// {data_j, seq, data_j+1, seq}.
//
// Validation: every lane checks its words' sequence numbers; a wavefront
// folds its 64 lanes' verdicts with one ballot per word slot.  When the whole
// wavefront is clean (the normal case) that is the only cost; otherwise the
// wave-uniform count and first index are accumulated in scalar registers and
// one lane issues two atomics when the wavefront retires.
#include "ar_device.hpp"
#include "ar_internal.hpp"

namespace ar {

namespace {

// Wave-uniform error record.
struct WaveErr {
  uint64_t count = 0;
  uint64_t first = ~0ull;
};

// Fold one word slot: `bad` per lane, `idx` this lane's word index (indices
// increase with the lane number, so the lowest flagged lane has the smallest
// index of this slot).
__device__ __forceinline__ void wave_note(WaveErr& e, bool bad, uint64_t idx) {
  const uint64_t m = __ballot(bad);
  if (m) {
    e.count += (uint64_t)__popcll(m);
    const int l = __ffsll((long long)m) - 1;
    const uint64_t fi = __shfl(idx, l);
    e.first = fi < e.first ? fi : e.first;
  }
}

__device__ __forceinline__ void wave_flush(const WaveErr& e, uint64_t* err) {
  if (e.count && lane_id() == 0) {
    atomicAdd(reinterpret_cast<unsigned long long*>(err), (unsigned long long)e.count);
    atomicMin(reinterpret_cast<unsigned long long*>(err + 1), (unsigned long long)e.first);
  }
}

// Base of this lane's wavefront in a grid-stride loop whose stride is a
// multiple of 64: every lane of a wavefront runs the same trip count, so the
// ballots always see the whole wavefront.
__device__ __forceinline__ size_t wave_base() {
  return (size_t)blockIdx.x * blockDim.x + (threadIdx.x & ~(kWave - 1));
}

}  // namespace

// ----------------------------------------------------------------------------
// Pack: 16 bytes of bf16 (4 data words) -> 32 bytes of payload.
template <bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void k_pack(const void* x, uint64_t* w, size_t n, uint32_t seq) {
  const size_t nvec = n >> 3;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const u32x4* src = static_cast<const u32x4*>(x);
  u32x4* dst = reinterpret_cast<u32x4*>(w);
  for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const u32x4 d = ld4<NTL>(src + v);
    u32x4 a, b;
    a[0] = d[0]; a[1] = seq; a[2] = d[1]; a[3] = seq;
    b[0] = d[2]; b[1] = seq; b[2] = d[3]; b[3] = seq;
    st4<NTS>(dst + 2 * v, a);
    st4<NTS>(dst + 2 * v + 1, b);
  }
  // tail: n is even, so 0..3 whole data words remain
  const size_t j = (nvec << 2) + threadIdx.x;
  if (blockIdx.x == 0 && j < (n >> 1)) {
    const uint32_t d = static_cast<const uint32_t*>(x)[j];
    w[j] = ((uint64_t)seq << 32) | (uint64_t)d;
  }
}

// Unpack + validate: 32 bytes of payload -> 16 bytes of bf16.
template <bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void k_unpack(const uint64_t* w, void* x, size_t n, uint32_t seq,
                                                   uint64_t* err) {
  const size_t nvec = n >> 3;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(w);
  u32x4* dst = static_cast<u32x4*>(x);
  WaveErr e;
  for (size_t base = wave_base(); base < nvec; base += stride) {
    const size_t v = base + lane_id();
    const bool act = v < nvec;
    u32x4 a = {0u, seq, 0u, seq}, b = {0u, seq, 0u, seq};
    if (act) {
      a = ld4<NTL>(src + 2 * v);
      b = ld4<NTL>(src + 2 * v + 1);
      u32x4 d;
      d[0] = a[0]; d[1] = a[2]; d[2] = b[0]; d[3] = b[2];
      st4<NTS>(dst + v, d);
    }
    const bool b0 = a[1] != seq, b1 = a[3] != seq, b2 = b[1] != seq, b3 = b[3] != seq;
    if (__ballot(b0 | b1 | b2 | b3)) {
      const uint64_t j = 4 * (uint64_t)v;
      wave_note(e, b0, j);
      wave_note(e, b1, j + 1);
      wave_note(e, b2, j + 2);
      wave_note(e, b3, j + 3);
    }
  }
  wave_flush(e, err);
  const size_t j = (nvec << 2) + threadIdx.x;
  if (blockIdx.x == 0 && j < (n >> 1)) {
    const uint64_t wj = w[j];
    static_cast<uint32_t*>(x)[j] = (uint32_t)wj;
    if ((uint32_t)(wj >> 32) != seq) {
      atomicAdd(reinterpret_cast<unsigned long long*>(err), 1ull);
      atomicMin(reinterpret_cast<unsigned long long*>(err + 1), (unsigned long long)j);
    }
  }
}

// ----------------------------------------------------------------------------
// Fused recursive doubling: one lane owns a 16-byte group (2 payload words,
// 4 bf16 elements) of every rank, checks every rank's sequence numbers, then
// runs all log2 P exchange steps in registers.  Step k combines rank r with
// r XOR 2^k; after step k ranks r and r XOR 2^k hold the same value, so the
// steps reduce to a balanced tree ((x0 x1)(x2 x3))((x4 x5)(x6 x7)) computed
// once per element and stored to all P outputs.  ROUND_EACH: every internal
// node is rounded to bf16, as the exchanged payload is bf16; otherwise the
// partials stay binary32 and are rounded once.
template <int P, bool ROUND_EACH, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void k_rd_fused(WordIn in, WordOut out, size_t W, uint32_t seq0,
                                                     uint64_t* err) {
  constexpr uint32_t L = P == 2 ? 1 : (P == 4 ? 2 : 3);
  const uint32_t seq_out = seq0 + L;
  const size_t nvec = W >> 1;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  WaveErr e;
  for (size_t base = wave_base(); base < nvec; base += stride) {
    const size_t v = base + lane_id();
    const bool act = v < nvec;
    u32x4 a[P];
    bool any = false;
    bool bad[P][2];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      a[p] = act ? ld4<NTL>(reinterpret_cast<const u32x4*>(in.p[p]) + v) : u32x4{0u, seq0, 0u, seq0};
      bad[p][0] = a[p][1] != seq0;
      bad[p][1] = a[p][3] != seq0;
      any |= bad[p][0] | bad[p][1];
    }
    if (__ballot(any)) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        wave_note(e, bad[p][0], (uint64_t)p * W + 2 * (uint64_t)v);
        wave_note(e, bad[p][1], (uint64_t)p * W + 2 * (uint64_t)v + 1);
      }
    }
    if (act) {
      float f[P][4];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        f[p][0] = lo_f32(a[p][0]);
        f[p][1] = hi_f32(a[p][0]);
        f[p][2] = lo_f32(a[p][2]);
        f[p][3] = hi_f32(a[p][2]);
      }
#pragma unroll
      for (int h = 1; h < P; h <<= 1) {
#pragma unroll
        for (int i = 0; i < P; i += 2 * h) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float s = f[i][k] + f[i + h][k];
            f[i][k] = ROUND_EACH ? round_bf16(s) : s;
          }
        }
      }
      u32x4 o;
      o[0] = pack_bf16x2(f[0][0], f[0][1]);
      o[1] = seq_out;
      o[2] = pack_bf16x2(f[0][2], f[0][3]);
      o[3] = seq_out;
#pragma unroll
      for (int p = 0; p < P; ++p) st4<NTS>(reinterpret_cast<u32x4*>(out.p[p]) + v, o);
    }
  }
  wave_flush(e, err);
  // odd word count: the last word, one lane
  if (blockIdx.x == 0 && threadIdx.x == 0 && (W & 1)) {
    const size_t j = W - 1;
    float f[P][2];
    for (int p = 0; p < P; ++p) {
      const uint64_t wj = in.p[p][j];
      if ((uint32_t)(wj >> 32) != seq0) {
        atomicAdd(reinterpret_cast<unsigned long long*>(err), 1ull);
        atomicMin(reinterpret_cast<unsigned long long*>(err + 1), (unsigned long long)(p * W + j));
      }
      f[p][0] = lo_f32((uint32_t)wj);
      f[p][1] = hi_f32((uint32_t)wj);
    }
    for (int h = 1; h < P; h <<= 1)
      for (int i = 0; i < P; i += 2 * h)
        for (int k = 0; k < 2; ++k) {
          const float s = f[i][k] + f[i + h][k];
          f[i][k] = ROUND_EACH ? round_bf16(s) : s;
        }
    const uint64_t o = ((uint64_t)seq_out << 32) | pack_bf16x2(f[0][0], f[0][1]);
    for (int p = 0; p < P; ++p) out.p[p][j] = o;
  }
}

// Staged recursive doubling, one launch per step k.  blockIdx.y picks the
// pair (r, q = r | 2^k) with bit k of r clear; a lane reads both payload
// groups, checks both sequence numbers (each payload of the step is received
// by exactly one partner, so each is checked once), adds, rounds, and writes
// the new payload to both ranks' destinations.  One lane per pair makes
// exact in-place aliasing safe.
template <bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void k_rd_step(WordIn src, WordOut dst, int P, int k, size_t W,
                                                    uint32_t seq_in, uint64_t* err) {
  const int i = blockIdx.y;
  const int low = i & ((1 << k) - 1);
  const int r = ((i >> k) << (k + 1)) | low;
  const int q = r | (1 << k);
  const uint32_t seq_out = seq_in + 1u;
  const size_t nvec = W >> 1;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const uint64_t base_r = ((uint64_t)k * P + r) * W;
  const uint64_t base_q = ((uint64_t)k * P + q) * W;
  const u32x4* sr = reinterpret_cast<const u32x4*>(src.p[r]);
  const u32x4* sq = reinterpret_cast<const u32x4*>(src.p[q]);
  u32x4* dr = reinterpret_cast<u32x4*>(dst.p[r]);
  u32x4* dq = reinterpret_cast<u32x4*>(dst.p[q]);
  WaveErr e;
  for (size_t base = wave_base(); base < nvec; base += stride) {
    const size_t v = base + lane_id();
    const bool act = v < nvec;
    u32x4 a = {0u, seq_in, 0u, seq_in}, b = a;
    if (act) {
      a = ld4<NTL>(sr + v);
      b = ld4<NTL>(sq + v);
    }
    const bool ba0 = a[1] != seq_in, ba1 = a[3] != seq_in, bb0 = b[1] != seq_in, bb1 = b[3] != seq_in;
    if (__ballot(ba0 | ba1 | bb0 | bb1)) {
      wave_note(e, ba0, base_r + 2 * (uint64_t)v);
      wave_note(e, ba1, base_r + 2 * (uint64_t)v + 1);
      wave_note(e, bb0, base_q + 2 * (uint64_t)v);
      wave_note(e, bb1, base_q + 2 * (uint64_t)v + 1);
    }
    if (act) {
      u32x4 o;
      o[0] = pack_bf16x2(lo_f32(a[0]) + lo_f32(b[0]), hi_f32(a[0]) + hi_f32(b[0]));
      o[1] = seq_out;
      o[2] = pack_bf16x2(lo_f32(a[2]) + lo_f32(b[2]), hi_f32(a[2]) + hi_f32(b[2]));
      o[3] = seq_out;
      st4<NTS>(dr + v, o);
      st4<NTS>(dq + v, o);
    }
  }
  wave_flush(e, err);
  if (blockIdx.x == 0 && threadIdx.x == 0 && (W & 1)) {
    const size_t j = W - 1;
    const uint64_t wa = src.p[r][j], wb = src.p[q][j];
    if ((uint32_t)(wa >> 32) != seq_in) {
      atomicAdd(reinterpret_cast<unsigned long long*>(err), 1ull);
      atomicMin(reinterpret_cast<unsigned long long*>(err + 1), (unsigned long long)(base_r + j));
    }
    if ((uint32_t)(wb >> 32) != seq_in) {
      atomicAdd(reinterpret_cast<unsigned long long*>(err), 1ull);
      atomicMin(reinterpret_cast<unsigned long long*>(err + 1), (unsigned long long)(base_q + j));
    }
    const uint32_t da = (uint32_t)wa, db = (uint32_t)wb;
    const uint64_t o = ((uint64_t)seq_out << 32) |
                       pack_bf16x2(lo_f32(da) + lo_f32(db), hi_f32(da) + hi_f32(db));
    dst.p[r][j] = o;
    dst.p[q][j] = o;
  }
}

__global__ void k_err_init(uint64_t* err) {
  if (threadIdx.x == 0) {
    err[0] = 0;
    err[1] = ~0ull;
  }
}

// ----------------------------------------------------------------------------
namespace {

inline unsigned grid_for(const Launch& L, size_t items) {
  const size_t want = cdiv(items, kBlock);
  const size_t cap = (size_t)L.cus * (size_t)L.grid_mult;
  const size_t g = want < cap ? want : cap;
  return (unsigned)(g ? g : 1);
}

inline int nt_mode(const Launch& L) { return (L.nt_loads ? 1 : 0) | (L.nt_stores ? 2 : 0); }

template <int P, bool RE>
hipError_t rd_fused_p(const Launch& L, const WordIn& in, const WordOut& out, size_t W, uint32_t seq0,
                      uint64_t* err) {
  const unsigned g = grid_for(L, W >> 1);
  switch (nt_mode(L)) {
    case 0: return launch_k(k_rd_fused<P, RE, false, false>, g, kBlock, L.stream, in, out, W, seq0, err);
    case 1: return launch_k(k_rd_fused<P, RE, true, false>, g, kBlock, L.stream, in, out, W, seq0, err);
    case 2: return launch_k(k_rd_fused<P, RE, false, true>, g, kBlock, L.stream, in, out, W, seq0, err);
    default: return launch_k(k_rd_fused<P, RE, true, true>, g, kBlock, L.stream, in, out, W, seq0, err);
  }
}

}  // namespace

hipError_t launch_pack(const Launch& L, const void* x, uint64_t* w, size_t n, uint32_t seq) {
  const unsigned g = grid_for(L, n >> 3);
  switch (nt_mode(L)) {
    case 0: return launch_k(k_pack<false, false>, g, kBlock, L.stream, x, w, n, seq);
    case 1: return launch_k(k_pack<true, false>, g, kBlock, L.stream, x, w, n, seq);
    case 2: return launch_k(k_pack<false, true>, g, kBlock, L.stream, x, w, n, seq);
    default: return launch_k(k_pack<true, true>, g, kBlock, L.stream, x, w, n, seq);
  }
}

hipError_t launch_unpack(const Launch& L, const uint64_t* w, void* x, size_t n, uint32_t seq,
                         uint64_t* d_err) {
  const unsigned g = grid_for(L, n >> 3);
  switch (nt_mode(L)) {
    case 0: return launch_k(k_unpack<false, false>, g, kBlock, L.stream, w, x, n, seq, d_err);
    case 1: return launch_k(k_unpack<true, false>, g, kBlock, L.stream, w, x, n, seq, d_err);
    case 2: return launch_k(k_unpack<false, true>, g, kBlock, L.stream, w, x, n, seq, d_err);
    default: return launch_k(k_unpack<true, true>, g, kBlock, L.stream, w, x, n, seq, d_err);
  }
}

hipError_t launch_rd_fused(const Launch& L, const WordIn& in, const WordOut& out, int P, size_t n,
                           uint32_t seq0, int fp32_carry, uint64_t* d_err) {
  const size_t W = n >> 1;
  if (fp32_carry) {
    switch (P) {
      case 2: return rd_fused_p<2, false>(L, in, out, W, seq0, d_err);
      case 4: return rd_fused_p<4, false>(L, in, out, W, seq0, d_err);
      case 8: return rd_fused_p<8, false>(L, in, out, W, seq0, d_err);
      default: return hipErrorInvalidValue;
    }
  }
  switch (P) {
    case 2: return rd_fused_p<2, true>(L, in, out, W, seq0, d_err);
    case 4: return rd_fused_p<4, true>(L, in, out, W, seq0, d_err);
    case 8: return rd_fused_p<8, true>(L, in, out, W, seq0, d_err);
    default: return hipErrorInvalidValue;
  }
}

size_t rd_mailbox_stride(size_t n) {
  const size_t W = n >> 1;
  return W + (W & 1);
}

hipError_t launch_rd_staged(const Launch& L, const WordIn& in, const WordOut& out, int P, size_t n,
                            uint32_t seq0, uint64_t* mailbox, uint64_t* d_err) {
  const size_t W = n >> 1;
  const size_t Ws = rd_mailbox_stride(n);
  const int steps = P == 2 ? 1 : (P == 4 ? 2 : 3);
  const unsigned gx = grid_for(L, W >> 1);
  const dim3 grid(gx > 0 ? (gx + (unsigned)(P / 2) - 1) / (unsigned)(P / 2) : 1, (unsigned)(P / 2));
  for (int k = 0; k < steps; ++k) {
    WordIn s{};
    WordOut d{};
    for (int r = 0; r < P; ++r) {
      s.p[r] = k == 0 ? in.p[r] : mailbox + ((size_t)(k - 1) * P + r) * Ws;
      d.p[r] = k == steps - 1 ? out.p[r] : mailbox + ((size_t)k * P + r) * Ws;
    }
    const uint32_t sk = seq0 + (uint32_t)k;
    hipError_t e;
    switch (nt_mode(L)) {
      case 0: e = launch_k(k_rd_step<false, false>, grid, kBlock, L.stream, s, d, P, k, W, sk, d_err); break;
      case 1: e = launch_k(k_rd_step<true, false>, grid, kBlock, L.stream, s, d, P, k, W, sk, d_err); break;
      case 2: e = launch_k(k_rd_step<false, true>, grid, kBlock, L.stream, s, d, P, k, W, sk, d_err); break;
      default: e = launch_k(k_rd_step<true, true>, grid, kBlock, L.stream, s, d, P, k, W, sk, d_err); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_err_init(const Launch& L, uint64_t* d_err) {
  return launch_k(k_err_init, dim3(1), dim3(kWave), L.stream, d_err);
}

}  // namespace ar
