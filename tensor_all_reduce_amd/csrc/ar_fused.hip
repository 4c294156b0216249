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
// folds its 64 lanes' flags with one ballot.  When the whole wavefront is
// clean (the normal case) that is the only cost; otherwise one ballot per
// word slot gives the wave-uniform count and first index, and one lane
// issues two atomics.
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

// One lane adds the wavefront's count and lowers the first index.  The
// stored minimum only ever decreases, so a relaxed read that already shows a
// value not above this wavefront's first index (a stale read can only show a
// larger one) makes the atomic minimum unnecessary: when every word is bad,
// this removes most of the atomics contending on err[1].
__device__ __forceinline__ void wave_flush(const WaveErr& e, uint64_t* err) {
  if (e.count && lane_id() == 0) {
    atomicAdd(reinterpret_cast<unsigned long long*>(err), (unsigned long long)e.count);
    if (e.first < __hip_atomic_load(err + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMin(reinterpret_cast<unsigned long long*>(err + 1), (unsigned long long)e.first);
  }
}

}  // namespace

// ----------------------------------------------------------------------------
// All kernels below use a flat grid: lane (blockIdx.x * blockDim.x + tid)
// owns a fixed run of payload words, workgroups dispatched in address order
// (the launch shape that measured fastest for streaming on MI355X).  The
// ragged end (the data words past the last whole run) is done by the last
// workgroup.
//
// Pack and unpack take the workgroup size as a template constant BLOCK for
// small messages (0: read blockDim and gridDim).  The kernel then reads no
// hidden dispatch arguments, its argument segment is its explicit arguments
// alone (32 and 40 bytes instead of 288 and 296), and HIP enqueues a kernel
// whose segment is at most 112 bytes about 0.7 us faster: the cost that
// bounds a decode-size call issued from the host.  The last workgroup is then
// computed from n, the same way the launcher sizes the grid.

// Pack: lane v turns data words [WPL*v, WPL*v + WPL) (WPL = 2: 8 bytes of
// bf16; 4: 16 bytes) into WPL payload words (16 or 32 bytes).  WPL = 2 makes
// every wavefront store instruction one contiguous 1 KiB: with WPL = 4 each
// lane stores two adjacent 16-byte groups, so each instruction covers a
// 2 KiB span half-filled, and that measured 8% slower.
// Whether this is the grid's last workgroup: from the template constant
// (grid = max(1, ceil(lanes / BLOCK)), as flat_grid sizes it) or from the
// dispatch.
template <int BLOCK>
__device__ __forceinline__ bool last_group(size_t lanes) {
  if constexpr (BLOCK > 0) return blockIdx.x == (unsigned)(lanes ? (lanes - 1) / BLOCK : 0);
  else return blockIdx.x == gridDim.x - 1;
}

template <int WPL, bool NTL, int SP, int BLOCK>
__global__ __launch_bounds__(BLOCK > 0 ? BLOCK : kMaxBlock) void k_pack(const void* x, uint64_t* w, size_t n,
                                                                        uint32_t seq) {
  const size_t nl = (n >> 1) / WPL;
  const unsigned nthr = BLOCK > 0 ? (unsigned)BLOCK : blockDim.x;
  const size_t v0 = (size_t)blockIdx.x * nthr;  // the workgroup's first lane
  const size_t v = v0 + threadIdx.x;
  if (v < nl) {
    u32x4* dst = reinterpret_cast<u32x4*>(w);
    if constexpr (WPL == 2) {
      const uint64_t d = ld8<NTL>(static_cast<const uint64_t*>(x) + v);
      u32x4 a;
      a[0] = (uint32_t)d; a[1] = seq; a[2] = (uint32_t)(d >> 32); a[3] = seq;
      st16<SP>(dst + v0, nthr * 16u, threadIdx.x * 16u, a);
    } else {
      const u32x4 d = ld4<NTL>(static_cast<const u32x4*>(x) + v);
      u32x4 a, b;
      a[0] = d[0]; a[1] = seq; a[2] = d[1]; a[3] = seq;
      b[0] = d[2]; b[1] = seq; b[2] = d[3]; b[3] = seq;
      st16<SP>(dst + 2 * v0, nthr * 32u, threadIdx.x * 32u, a);
      st16<SP>(dst + 2 * v0, nthr * 32u, threadIdx.x * 32u + 16u, b);
    }
  }
  // tail: n is even, so fewer than WPL whole data words remain
  const size_t j = nl * WPL + threadIdx.x;
  if (last_group<BLOCK>(nl) && j < (n >> 1)) {
    const uint32_t d = static_cast<const uint32_t*>(x)[j];
    w[j] = ((uint64_t)seq << 32) | (uint64_t)d;
  }
}

// Unpack + validate: lane v reads payload words [WPL*v, WPL*v + WPL) and
// writes their data words (WPL = 2: one 16-byte load, one 8-byte store, each
// wavefront instruction contiguous; WPL = 4: two adjacent 16-byte loads).
template <int WPL, bool NTL, int SP, int BLOCK>
__global__ __launch_bounds__(BLOCK > 0 ? BLOCK : kMaxBlock) void k_unpack(const uint64_t* w, void* x, size_t n,
                                                                          uint32_t seq, uint64_t* err) {
  const size_t nl = (n >> 1) / WPL;
  const unsigned nthr = BLOCK > 0 ? (unsigned)BLOCK : blockDim.x;
  const size_t v0 = (size_t)blockIdx.x * nthr;
  const size_t v = v0 + threadIdx.x;
  const bool act = v < nl;
  const u32x4* src = reinterpret_cast<const u32x4*>(w);
  u32x4 a = {0u, seq, 0u, seq}, b = {0u, seq, 0u, seq};
  if (act) {
    if constexpr (WPL == 2) {
      a = ld4<NTL>(src + v);
      st8p<SP>(static_cast<uint64_t*>(x) + v0, nthr * 8u, threadIdx.x * 8u,
               (uint64_t)a[0] | ((uint64_t)a[2] << 32));
    } else {
      a = ld4<NTL>(src + 2 * v);
      b = ld4<NTL>(src + 2 * v + 1);
      u32x4 d;
      d[0] = a[0]; d[1] = a[2]; d[2] = b[0]; d[3] = b[2];
      st16<SP>(static_cast<u32x4*>(x) + v0, nthr * 16u, threadIdx.x * 16u, d);
    }
  }
  const bool b0 = a[1] != seq, b1 = a[3] != seq, b2 = b[1] != seq, b3 = b[3] != seq;
  WaveErr e;
  if (__ballot(b0 | b1 | b2 | b3)) {
    const uint64_t j = WPL * (uint64_t)v;
    wave_note(e, b0, j);
    wave_note(e, b1, j + 1);
    if constexpr (WPL == 4) {
      wave_note(e, b2, j + 2);
      wave_note(e, b3, j + 3);
    }
  }
  wave_flush(e, err);
  const size_t j = nl * WPL + threadIdx.x;
  if (last_group<BLOCK>(nl) && j < (n >> 1)) {
    const uint64_t wj = w[j];
    static_cast<uint32_t*>(x)[j] = (uint32_t)wj;
    if ((uint32_t)(wj >> 32) != seq) {
      atomicAdd(reinterpret_cast<unsigned long long*>(err), 1ull);
      atomicMin(reinterpret_cast<unsigned long long*>(err + 1), (unsigned long long)j);
    }
  }
}

// ----------------------------------------------------------------------------
// Fused recursive doubling: one lane owns V 16-byte groups (2 payload words,
// 4 bf16 elements each) of every rank, checks every rank's sequence numbers, then
// runs all log2 P exchange steps in registers.  Step k combines rank r with
// r XOR 2^k; after step k ranks r and r XOR 2^k hold the same value, so the
// steps reduce to a balanced tree ((x0 x1)(x2 x3))((x4 x5)(x6 x7)) computed
// once per element and stored to all P outputs.  ROUND_EACH: every internal
// node is rounded to bf16, as the exchanged payload is bf16; otherwise the
// partials stay binary32 and are rounded once.
template <int P, int V, bool ROUND_EACH, bool NTL, int SP>
__global__ __launch_bounds__(kMaxBlock) void k_rd_fused(WordIn in, WordOut out, size_t W, uint32_t seq0,
                                                       uint64_t* err) {
  constexpr uint32_t L = P == 2 ? 1 : (P == 4 ? 2 : 3);
  const uint32_t seq_out = seq0 + L;
  const size_t nvec = W >> 1;
  // a workgroup owns V * blockDim consecutive groups; all V * P loads are
  // issued before any arithmetic
  const size_t wg0 = (size_t)blockIdx.x * V * blockDim.x;  // the workgroup's first group
  const size_t base = wg0 + threadIdx.x;
  u32x4 a[V][P];
  bool any = false;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t v = base + (size_t)u * blockDim.x;
    const bool act = v < nvec;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      a[u][p] = act ? ld4<NTL>(reinterpret_cast<const u32x4*>(in.p[p]) + v) : u32x4{0u, seq0, 0u, seq0};
      any |= (a[u][p][1] != seq0) | (a[u][p][3] != seq0);
    }
  }
  WaveErr e;
  if (__ballot(any)) {
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const uint64_t v = base + (uint64_t)u * blockDim.x;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        wave_note(e, a[u][p][1] != seq0, (uint64_t)p * W + 2 * v);
        wave_note(e, a[u][p][3] != seq0, (uint64_t)p * W + 2 * v + 1);
      }
    }
  }
  wave_flush(e, err);
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const size_t v = base + (size_t)u * blockDim.x;
    if (v < nvec) {
      float f[P][4];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        f[p][0] = lo_f32(a[u][p][0]);
        f[p][1] = hi_f32(a[u][p][0]);
        f[p][2] = lo_f32(a[u][p][2]);
        f[p][3] = hi_f32(a[u][p][2]);
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
      for (int p = 0; p < P; ++p)
        st16<SP>(reinterpret_cast<u32x4*>(out.p[p]) + wg0, (uint32_t)V * blockDim.x * 16u,
                 (uint32_t)(v - wg0) * 16u, o);
    }
  }
  // odd word count: the last word, one lane
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0 && (W & 1)) {
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

// Staged recursive doubling, one launch per step k.  Workgroup b works on
// tile b / (P/2) of pair b % (P/2), so consecutive workgroups cover every
// pair at the same offset and all P payload streams advance together.  The
// pair (r, q = r | 2^k) has bit k of r clear; a lane reads both payload
// groups, checks both sequence numbers (each payload of the step is received
// by exactly one partner, so each is checked once), adds, rounds, and writes
// the new payload to both ranks' destinations.  One lane per pair makes
// exact in-place aliasing safe.
template <bool NTL, int SP>
__global__ __launch_bounds__(kMaxBlock) void k_rd_step(WordIn src, WordOut dst, int P, int k, size_t W,
                                                      uint32_t seq_in, uint64_t* err) {
  const unsigned npairs = (unsigned)P >> 1;
  const int i = (int)(blockIdx.x % npairs);
  const size_t tile = blockIdx.x / npairs;
  const size_t ntiles = gridDim.x / npairs;
  const int low = i & ((1 << k) - 1);
  const int r = ((i >> k) << (k + 1)) | low;
  const int q = r | (1 << k);
  const uint32_t seq_out = seq_in + 1u;
  const size_t nvec = W >> 1;
  const uint64_t base_r = ((uint64_t)k * P + r) * W;
  const uint64_t base_q = ((uint64_t)k * P + q) * W;
  const size_t v = tile * blockDim.x + threadIdx.x;
  const bool act = v < nvec;
  u32x4 a = {0u, seq_in, 0u, seq_in}, b = a;
  if (act) {
    a = ld4<NTL>(reinterpret_cast<const u32x4*>(src.p[r]) + v);
    b = ld4<NTL>(reinterpret_cast<const u32x4*>(src.p[q]) + v);
  }
  const bool ba0 = a[1] != seq_in, ba1 = a[3] != seq_in, bb0 = b[1] != seq_in, bb1 = b[3] != seq_in;
  WaveErr e;
  if (__ballot(ba0 | ba1 | bb0 | bb1)) {
    wave_note(e, ba0, base_r + 2 * (uint64_t)v);
    wave_note(e, ba1, base_r + 2 * (uint64_t)v + 1);
    wave_note(e, bb0, base_q + 2 * (uint64_t)v);
    wave_note(e, bb1, base_q + 2 * (uint64_t)v + 1);
  }
  wave_flush(e, err);
  if (act) {
    u32x4 o;
    o[0] = pack_bf16x2(lo_f32(a[0]) + lo_f32(b[0]), hi_f32(a[0]) + hi_f32(b[0]));
    o[1] = seq_out;
    o[2] = pack_bf16x2(lo_f32(a[2]) + lo_f32(b[2]), hi_f32(a[2]) + hi_f32(b[2]));
    o[3] = seq_out;
    const size_t t0 = tile * blockDim.x;
    st16<SP>(reinterpret_cast<u32x4*>(dst.p[r]) + t0, blockDim.x * 16u, threadIdx.x * 16u, o);
    st16<SP>(reinterpret_cast<u32x4*>(dst.p[q]) + t0, blockDim.x * 16u, threadIdx.x * 16u, o);
  }
  if (tile == ntiles - 1 && threadIdx.x == 0 && (W & 1)) {
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

// ----------------------------------------------------------------------------
// Unpack with a bounded wait for a concurrent producer.  Each payload word is
// read with a 64-bit agent-scope atomic load: the data and its sequence
// number are one naturally aligned 8-byte word, so a load that returns the
// expected sequence number returns that word's data with it (the producer's
// stores write whole aligned words).  Persistent grid: wavefront q of Q owns
// the 256-word tiles q, q + Q, ...; its k-th load instruction reads words
// tile + 64k + lane, so every load (512 bytes) and every data store (256
// bytes) of a wavefront is one contiguous span.  `spins` is the wavefront's
// total poll budget across all its tiles, which bounds the kernel's run time
// even when the producer never comes.
__device__ __forceinline__ uint64_t ld_word_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool NTS>
__global__ __launch_bounds__(kMaxBlock) void k_unpack_wait(const uint64_t* w, void* x, size_t n, uint32_t seq,
                                                          uint32_t max_spins, uint64_t* err) {
  constexpr int K = 4;                          // words per lane per tile
  const size_t W = n >> 1;
  const size_t wave = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const size_t nwaves = (size_t)gridDim.x * blockDim.x / kWave;
  const uint32_t lane = lane_id();
  uint32_t* x32 = static_cast<uint32_t*>(x);
  uint32_t spins = 0;
  WaveErr e;
  for (size_t tile = wave * (K * kWave); tile < W; tile += nwaves * (K * kWave)) {
    uint64_t q[K];
    bool ok = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const size_t j = tile + (size_t)k * kWave + lane;
      q[k] = j < W ? ld_word_agent(w + j) : ((uint64_t)seq << 32);
      ok = ok && (uint32_t)(q[k] >> 32) == seq;
    }
    while (__ballot(!ok) && spins < max_spins) {
      __builtin_amdgcn_s_sleep(1);
      ++spins;
      if (!ok) {
        ok = true;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const size_t j = tile + (size_t)k * kWave + lane;
          if ((uint32_t)(q[k] >> 32) != seq) q[k] = ld_word_agent(w + j);
          ok = ok && (uint32_t)(q[k] >> 32) == seq;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const size_t j = tile + (size_t)k * kWave + lane;
      if (j < W) {
        if constexpr (NTS) __builtin_nontemporal_store((uint32_t)q[k], x32 + j);
        else x32[j] = (uint32_t)q[k];
      }
    }
    if (__ballot(!ok)) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const size_t j = tile + (size_t)k * kWave + lane;
        wave_note(e, (uint32_t)(q[k] >> 32) != seq, (uint64_t)j);
      }
    }
  }
  wave_flush(e, err);
}

__global__ void k_err_init(uint64_t* err) {
  if (threadIdx.x == 0) {
    err[0] = 0;
    err[1] = ~0ull;
  }
}

// ----------------------------------------------------------------------------
namespace {

// Flat grid: one lane per 16-byte group, at least one workgroup (the last
// workgroup also does the ragged end).
inline unsigned flat_grid(const Shape& sh, size_t items) {
  const size_t g = cdiv(items, (size_t)sh.block);
  return (unsigned)(g ? g : 1);
}

inline bool grid_fits(const Shape& sh, size_t items) {
  return cdiv(items, (size_t)sh.block) <= 0x7FFFFFFFull;
}

template <int P, int V, bool RE>
hipError_t rd_fused_v(const Shape& sh, hipStream_t st, const WordIn& in, const WordOut& out, size_t W,
                      uint32_t seq0, uint64_t* err) {
  const size_t gs = cdiv(W >> 1, (size_t)V * sh.block);
  const unsigned g = (unsigned)(gs ? gs : 1);
  const dim3 b(sh.block);
  return with_policy(sh, [&](auto ntl, auto sp) {
    return launch_k(k_rd_fused<P, V, RE, decltype(ntl)::value, decltype(sp)::value>, g, b, sh.lds, st, in, out, W,
                    seq0, err);
  });
}

template <int P, bool RE>
hipError_t rd_fused_p(const Launch& L, const WordIn& in, const WordOut& out, size_t W, uint32_t seq0,
                      uint64_t* err) {
  const Shape& sh = shape_for(L, kRD, kRDSmall, 2 * W);
  if (sh.vec == 2) return rd_fused_v<P, 2, RE>(sh, L.stream, in, out, W, seq0, err);
  return rd_fused_v<P, 1, RE>(sh, L.stream, in, out, W, seq0, err);
}

}  // namespace

template <int WPL>
hipError_t pack_w(const Shape& sh, hipStream_t st, const void* x, uint64_t* w, size_t n, uint32_t seq,
                  bool small) {
  const size_t nl = (n >> 1) / WPL;
  if (!grid_fits(sh, nl)) return hipErrorInvalidConfiguration;
  const unsigned g = flat_grid(sh, nl);
  auto go = [&](auto blk) {
    return with_policy(sh, [&](auto ntl, auto sp) {
      return launch_k(k_pack<WPL, decltype(ntl)::value, decltype(sp)::value, decltype(blk)::value>, g,
                      dim3(sh.block), sh.lds, st, x, w, n, seq);
    });
  };
  if (small && sh.block == 64) return go(SPc<64>{});
  if (small && sh.block == 128) return go(SPc<128>{});
  if (small && sh.block == 256) return go(SPc<256>{});
  return go(SPc<0>{});
}

template <int WPL>
hipError_t unpack_w(const Shape& sh, hipStream_t st, const uint64_t* w, void* x, size_t n, uint32_t seq,
                    uint64_t* d_err, bool small) {
  const size_t nl = (n >> 1) / WPL;
  if (!grid_fits(sh, nl)) return hipErrorInvalidConfiguration;
  const unsigned g = flat_grid(sh, nl);
  auto go = [&](auto blk) {
    return with_policy(sh, [&](auto ntl, auto sp) {
      return launch_k(k_unpack<WPL, decltype(ntl)::value, decltype(sp)::value, decltype(blk)::value>, g,
                      dim3(sh.block), sh.lds, st, w, x, n, seq, d_err);
    });
  };
  if (small && sh.block == 64) return go(SPc<64>{});
  if (small && sh.block == 128) return go(SPc<128>{});
  if (small && sh.block == 256) return go(SPc<256>{});
  return go(SPc<0>{});
}

// For pack and unpack the shape's vec counts 16-byte groups of bf16 per lane:
// 1 -> 2 data words (8 bytes) per lane, 2 -> 4 data words (16 bytes).
hipError_t launch_pack(const Launch& L, const void* x, uint64_t* w, size_t n, uint32_t seq) {
  const bool small = n <= (size_t)AR_SMALL_ELEMS;
  const Shape& sh = small ? L.shape[kPackSmall] : L.shape[kPack];
  if (sh.vec == 2) return pack_w<4>(sh, L.stream, x, w, n, seq, small);
  return pack_w<2>(sh, L.stream, x, w, n, seq, small);
}

hipError_t launch_unpack(const Launch& L, const uint64_t* w, void* x, size_t n, uint32_t seq,
                         uint64_t* d_err) {
  const bool small = n <= (size_t)AR_SMALL_ELEMS;
  const Shape& sh = small ? L.shape[kUnpackSmall] : L.shape[kUnpack];
  if (sh.vec == 2) return unpack_w<4>(sh, L.stream, w, x, n, seq, d_err, small);
  return unpack_w<2>(sh, L.stream, w, x, n, seq, d_err, small);
}

hipError_t launch_rd_fused(const Launch& L, const WordIn& in, const WordOut& out, int P, size_t n,
                           uint32_t seq0, int fp32_carry, uint64_t* d_err) {
  const size_t W = n >> 1;
  if (!grid_fits(shape_for(L, kRD, kRDSmall, n), W >> 1)) return hipErrorInvalidConfiguration;
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
  const Shape& sh = shape_for(L, kRDStep, kRDStepSmall, n);
  const size_t tiles = flat_grid(sh, W >> 1);
  if (tiles * (size_t)(P / 2) > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(tiles * (size_t)(P / 2)));
  const dim3 b(sh.block);
  for (int k = 0; k < steps; ++k) {
    WordIn s{};
    WordOut d{};
    for (int r = 0; r < P; ++r) {
      s.p[r] = k == 0 ? in.p[r] : mailbox + ((size_t)(k - 1) * P + r) * Ws;
      d.p[r] = k == steps - 1 ? out.p[r] : mailbox + ((size_t)k * P + r) * Ws;
    }
    const uint32_t sk = seq0 + (uint32_t)k;
    const hipError_t e = with_policy(sh, [&](auto ntl, auto sp) {
      return launch_k(k_rd_step<decltype(ntl)::value, decltype(sp)::value>, grid, b, sh.lds, L.stream, s, d, P, k, W,
                      sk, d_err);
    });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_unpack_wait(const Launch& L, const uint64_t* w, void* x, size_t n, uint32_t seq,
                              uint32_t max_spins, uint64_t* d_err) {
  const Shape& sh = L.shape[kUnpackWait];
  // one 256-word tile per wavefront is enough to cover the buffer
  const size_t need = cdiv(cdiv(n >> 1, (size_t)4 * kWave), (size_t)sh.block / kWave);
  size_t g = (size_t)L.cus * (size_t)(sh.wg_per_cu > 0 ? sh.wg_per_cu : 1);
  if (g > need) g = need;
  if (g == 0) g = 1;
  const dim3 b(sh.block);
  // no LDS request here: the producer's workgroups must always fit beside these
  if (sh.stores & 1) return launch_k(k_unpack_wait<true>, (unsigned)g, b, 0, L.stream, w, x, n, seq, max_spins, d_err);
  return launch_k(k_unpack_wait<false>, (unsigned)g, b, 0, L.stream, w, x, n, seq, max_spins, d_err);
}

hipError_t launch_err_init(const Launch& L, uint64_t* d_err) {
  return launch_k(k_err_init, dim3(1), dim3(kWave), 0, L.stream, d_err);
}

}  // namespace ar
