// C-ABI of the all-reduce core (declared in include/ar.h): argument checks,
// the per-device attribute cache, tuning knobs, and dispatch to the kernels.
//
// Every argument check and every grid-size check runs before the first
// launch, so an argument error never leaves partial work queued.  The only
// global state is one immutable launch table per device (CU count and the
// resolved launch shapes), built on the first call on that device under a
// mutex and published through an atomic pointer: two host threads (one per
// ubatch) racing the first call must not both initialise it -- the
// lazy-initialisation race the review of "[DSV4] perf(tbo): overlap pure-TP
// all_reduce on TBO + Delay TP" flags for its per-ubatch communicators --
// and after that first call no call takes a lock.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "ar.h"
#include "ar_internal.hpp"

namespace ar {
size_t rd_mailbox_stride(size_t n);
}

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxUbatch = 16;

// Default launch shapes: the fastest settings measured on MI355X for each
// kernel's stream pattern (block, vec, nt_loads, stores, wg_per_cu; stores is
// the output store policy of st16: 0 plain, 1 NT, 2 SC1, 3 SC1 + NT).  For
// the one-shot and fused two-stage kernels, whose best shape for one
// placement of the rank buffers can lose 15-20% on another (buffers carved
// from one allocation, or halves of larger tensors), the pick is the shape
// with the best worst case over placements, within 1% of the best for
// separately allocated buffers.
constexpr ar::Shape kDefaultShape[] = {
    {64, 1, 1, 1, 8, 0},    // one-shot, 8 -> 1
    {64, 1, 1, 2, 6, 0},    // fused two-stage, 8 -> 8
    {64, 1, 1, 3, 6, 0},    // ubatch, 8 -> 8 on two streams
    {64, 1, 1, 2, 10, 0},   // staged reduce-scatter, 8 -> 1
    {64, 1, 0, 1, 3, 0},    // staged all-gather, 1 -> 8 (plain loads of scratch)
    {64, 1, 1, 3, 0, 0},    // pack, 1 -> 2 (vec: 16-byte bf16 groups per lane; 1 = 8 bytes);
                            // SC1 stores: a waiting receiver on another XCD sees each word once stored
    {64, 1, 1, 3, 0, 0},    // unpack, 2 -> 1
    {64, 1, 1, 3, 8, 0},    // fused recursive doubling, 8 -> 8
    {64, 1, 1, 2, 16, 0},   // staged recursive-doubling step, 8 -> 8
    {256, 1, 0, 1, 3, 0},   // waiting unpack: 3 persistent workgroups (12 waves) per CU
    {256, 1, 1, 3, 3, 0},   // flagged ubatch: big tiles, few store waits and counter atomics per chunk
    {64, 2, 1, 3, 0, 0},    // fp8 quantise, 1 -> 1 + scales, buffer after buffer
    {256, 1, 1, 1, 6, 0},   // fp8 reduce, P code streams -> 1 output (vec: 16-byte output groups per lane)
    {256, 1, 1, 3, 3, 0},   // fp8 reduce, P code streams -> P outputs
    {128, 1, 0, 2, 0, 0},   // one-shot, n <= AR_SMALL_ELEMS: uncapped, plain loads, SC1 stores
    {64, 1, 0, 2, 0, 0},    // fused two-stage, n <= AR_SMALL_ELEMS (its compact kernel takes buffer offsets)
    {64, 1, 0, 2, 0, 0},    // fused recursive doubling, n <= AR_SMALL_ELEMS
    {64, 1, 0, 0, 0, 0},    // staged RD step, n <= AR_SMALL_ELEMS: plain stores keep the mailbox on chip
    {256, 1, 0, 3, 0, 0},   // pack, n <= AR_SMALL_ELEMS: plain loads, uncapped, SC1 stores
    {256, 1, 0, 2, 0, 0},   // unpack, n <= AR_SMALL_ELEMS
    {512, 1, 1, 1, 4, 0},   // bounded ubatch: 512-lane workgroups on 4/8 of the CUs (wg_per_cu: eighths)
    {128, 1, 1, 1, 0, 0},   // in-place fused two-stage, n <= AR_SMALL_ELEMS: NT loads, so the NT stores
                            // that rewrite the same lines find them marked streaming
};
constexpr const char* kShapeEnv[] = {
    "AR_SHAPE_ONESHOT", "AR_SHAPE_2STAGE", "AR_SHAPE_UBATCH", "AR_SHAPE_RS", "AR_SHAPE_AG",
    "AR_SHAPE_PACK", "AR_SHAPE_UNPACK", "AR_SHAPE_RD", "AR_SHAPE_RDSTEP", "AR_SHAPE_UNPACK_WAIT",
    "AR_SHAPE_UBATCH_FLAGS", "AR_SHAPE_QUANT_FP8", "AR_SHAPE_REDUCE_FP8", "AR_SHAPE_REDUCE_FP8_ALL",
    "AR_SHAPE_ONESHOT_SMALL", "AR_SHAPE_2STAGE_SMALL", "AR_SHAPE_RD_SMALL", "AR_SHAPE_RDSTEP_SMALL",
    "AR_SHAPE_PACK_SMALL", "AR_SHAPE_UNPACK_SMALL", "AR_SHAPE_UBATCH_BOUNDED",
    "AR_SHAPE_2STAGE_INPLACE_SMALL"};
// one default and one override name per kind, in the order of ar.h's kind
// numbers
static_assert(sizeof(kDefaultShape) / sizeof(kDefaultShape[0]) == ar::kKinds, "a default shape per kind");
static_assert(sizeof(kShapeEnv) / sizeof(kShapeEnv[0]) == ar::kKinds, "an override name per kind");
static_assert(ar::kOneshot == AR_KERNEL_ONESHOT && ar::k2Stage == AR_KERNEL_2STAGE &&
                  ar::kUbatch == AR_KERNEL_UBATCH && ar::kRS == AR_KERNEL_RS && ar::kAG == AR_KERNEL_AG &&
                  ar::kPack == AR_KERNEL_PACK && ar::kUnpack == AR_KERNEL_UNPACK && ar::kRD == AR_KERNEL_RD &&
                  ar::kRDStep == AR_KERNEL_RDSTEP && ar::kUnpackWait == AR_KERNEL_UNPACK_WAIT &&
                  ar::kUbatchFlags == AR_KERNEL_UBATCH_FLAGS && ar::kQuantFp8 == AR_KERNEL_QUANT_FP8 &&
                  ar::kReduceFp8 == AR_KERNEL_REDUCE_FP8 && ar::kReduceFp8All == AR_KERNEL_REDUCE_FP8_ALL &&
                  ar::kOneshotSmall == AR_KERNEL_ONESHOT_SMALL && ar::k2StageSmall == AR_KERNEL_2STAGE_SMALL &&
                  ar::kRDSmall == AR_KERNEL_RD_SMALL && ar::kRDStepSmall == AR_KERNEL_RDSTEP_SMALL &&
                  ar::kPackSmall == AR_KERNEL_PACK_SMALL && ar::kUnpackSmall == AR_KERNEL_UNPACK_SMALL &&
                  ar::kUbatchBounded == AR_KERNEL_UBATCH_BOUNDED &&
                  ar::k2StageInplaceSmall == AR_KERNEL_2STAGE_INPLACE_SMALL &&
                  ar::kKinds == AR_KERNEL_2STAGE_INPLACE_SMALL + 1,
              "kind numbers match ar.h");

// What one device's calls read: its CU count and the launch shapes with
// their LDS requests resolved for it.  Never modified once published.
struct Table {
  int cus;
  void* scratch;  // device address of the static scratch array (nullptr: unavailable)
  ar::Shape shape[ar::kKinds];
};

// Scratch of ar_reduce_2stage_static.  In host code this name is only a
// stand-in for the symbol: each device's address of the array comes from
// hipGetSymbolAddress (stored in DevAttr::scratch / Table::scratch), and only
// that address is ever passed to a kernel.
static __device__ __align__(256) uint16_t scratch[AR_STATIC_SCRATCH_ELEMS];

struct DevAttr {
  int cus = 0, lds_per_cu = 0, lds_per_block = 0;
  void* scratch = nullptr;  // this device's address of the static scratch array
};

std::mutex g_mu;                              // initialisation and shape changes
bool g_base_ready = false;                    // guarded by g_mu
ar::Shape g_base[ar::kKinds];                 // defaults + overrides; guarded by g_mu
DevAttr g_attr[kMaxDevices];                  // guarded by g_mu
// Published tables are never freed: a call may still be reading a table that
// ar_set_launch_shape has replaced.  A device's first table is static
// storage, so no compute entry point allocates memory of any kind; only
// ar_set_launch_shape (a tuning knob) allocates a replacement table, ~500
// bytes, per device in use.
Table g_first_table[kMaxDevices];             // written once, under g_mu, before publication
std::atomic<const Table*> g_table[kMaxDevices];

bool shape_ok(int kind, int block, int vec, int ntl, int stores, int wg) {
  const bool fields = vec >= 1 && vec <= 2 && ntl >= 0 && ntl <= 1 && stores >= 0 && stores <= 3;
  if (kind == ar::kUbatchBounded)  // a persistent grid: 256..1024 lanes, wg counts eighths of the CUs
    return fields && (block == 256 || block == 512 || block == 1024) && wg >= 1 && wg <= 8;
  return fields && (block == 64 || block == 128 || block == 256) && wg >= 0 && wg <= 64;
}

// "block,vec,nt_loads,stores,wg_per_cu"; an invalid string keeps the default.
void parse_shape(int kind, const char* name, ar::Shape* s) {
  const char* e = std::getenv(name);
  if (!e || !*e) return;
  int v[5];
  if (std::sscanf(e, "%d,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3], &v[4]) != 5) return;
  if (!shape_ok(kind, v[0], v[1], v[2], v[3], v[4])) return;
  *s = ar::Shape{v[0], v[1], v[2], v[3], v[4], 0};
}

// Caller holds g_mu.
void init_base_locked() {
  if (g_base_ready) return;
  for (int k = 0; k < ar::kKinds; ++k) {
    g_base[k] = kDefaultShape[k];
    parse_shape(k, kShapeEnv[k], &g_base[k]);
  }
  g_base_ready = true;
}

// Build and publish device `dev`'s table from g_base: the device's first
// table into its static slot, a replacement on the heap.  Caller holds g_mu
// and has filled g_attr[dev].
const Table* publish_locked(int dev, bool first) {
  const DevAttr& d = g_attr[dev];
  Table* t = first ? &g_first_table[dev] : new Table;
  t->cus = d.cus;
  t->scratch = d.scratch;
  for (int k = 0; k < ar::kKinds; ++k) {
    ar::Shape s = g_base[k];
    unsigned lds = 0;
    if (s.wg_per_cu > 0 && d.lds_per_cu > 0 && k != ar::kUbatchBounded) {
      lds = ((unsigned)d.lds_per_cu / (unsigned)s.wg_per_cu) & ~255u;
      if (lds > (unsigned)d.lds_per_block) lds = (unsigned)d.lds_per_block;
    }
    s.lds = lds;
    t->shape[k] = s;
  }
  g_table[dev].store(t, std::memory_order_release);
  return t;
}

// Resolve the launch policy for the current device.  The first call on a
// device queries its attributes and builds its table under g_mu; every later
// call is one acquire load.  Shapes come from the defaults above, overridable
// once per process through AR_SHAPE_<KIND> or at any time through
// ar_set_launch_shape.
int resolve(ar::Launch* L, void* stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AR_ERR_HIP;
  const Table* t = g_table[dev].load(std::memory_order_acquire);
  if (!t) {
    std::lock_guard<std::mutex> lock(g_mu);
    t = g_table[dev].load(std::memory_order_relaxed);
    if (!t) {
      int cus = 0, lcu = 0, lblk = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          hipDeviceGetAttribute(&lcu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
              hipSuccess ||
          hipDeviceGetAttribute(&lblk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
          cus <= 0)
        return AR_ERR_HIP;
      // the static scratch array's address on this device (the device is
      // current here); a failure leaves it unavailable to the one entry
      // point that needs it and is reported there
      void* sp = nullptr;
      if (hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) != hipSuccess) {
        sp = nullptr;
        (void)hipGetLastError();
      }
      g_attr[dev] = DevAttr{cus, lcu, lblk, sp};
      init_base_locked();
      t = publish_locked(dev, true);
    }
  }
  L->cus = t->cus;
  L->shape = t->shape;
  L->scratch = t->scratch;
  L->stream = static_cast<hipStream_t>(stream);
  return AR_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

// A range that would run past the top of the address space (an impossible
// buffer, but a wrapped end would hide an overlap) ends at the top.
inline Span span_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uintptr_t room = ~(uintptr_t)0 - a;
  return Span{a, bytes > room ? ~(uintptr_t)0 : a + bytes};
}

inline bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }
inline bool same(Span a, Span b) { return a.lo == b.lo && a.hi == b.hi; }

// An output may coincide exactly with an input; any other overlap with an
// input is a partial alias.  Outputs may not overlap each other at all.
int check_outputs(const Span* ins, int nin, const Span* outs, int nout) {
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlap(outs[o], ins[i]) && !same(outs[o], ins[i])) return AR_ERR_ALIAS;
    for (int q = o + 1; q < nout; ++q)
      if (overlap(outs[o], outs[q])) return AR_ERR_ALIAS;
  }
  return AR_OK;
}

int check_disjoint(Span s, const Span* others, int k) {
  for (int i = 0; i < k; ++i)
    if (overlap(s, others[i])) return AR_ERR_ALIAS;
  return AR_OK;
}

bool mul_overflows(size_t a, size_t b) { return a != 0 && b > (~(size_t)0) / a; }

int hip_status(hipError_t e) { return e == hipSuccess ? AR_OK : AR_ERR_HIP; }

int check_ranks(const void* const* ins, int P, size_t n, ar::InPtrs* in, Span* spans) {
  if (!ins || P < 1 || P > AR_MAX_RANKS) return AR_ERR_INVALID;
  if (mul_overflows(n, 2)) return AR_ERR_INVALID;
  for (int p = 0; p < P; ++p) {
    if (!ins[p]) return AR_ERR_INVALID;
    if (!aligned16(ins[p])) return AR_ERR_ALIGN;
    in->p[p] = ins[p];
    spans[p] = span_of(ins[p], n * 2);
  }
  return AR_OK;
}

int check_err(const uint64_t* d_err) {
  if (!d_err) return AR_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(d_err) & 7u) return AR_ERR_ALIGN;
  return AR_OK;
}

}  // namespace

extern "C" {

const char* ar_status_str(int status) {
  switch (status) {
    case AR_OK: return "AR_OK";
    case AR_ERR_INVALID: return "AR_ERR_INVALID: invalid argument";
    case AR_ERR_ALIGN: return "AR_ERR_ALIGN: pointer not 16-byte aligned";
    case AR_ERR_ALIAS: return "AR_ERR_ALIAS: buffers partially overlap";
    case AR_ERR_UNSUPPORTED: return "AR_ERR_UNSUPPORTED: unsupported configuration";
    case AR_ERR_HIP: return "AR_ERR_HIP: HIP runtime or launch failure";
    case AR_ERR_SIZE: return "AR_ERR_SIZE: n exceeds AR_STATIC_SCRATCH_ELEMS, the static scratch";
    default: return "AR_ERR_UNKNOWN";
  }
}

int ar_version(void) { return 10000; }

int ar_reduce_oneshot(const void* const* ins, int P, void* out, size_t n, void* stream) {
  ar::InPtrs in{};
  Span si[AR_MAX_RANKS];
  int rc = check_ranks(ins, P, n, &in, si);
  if (rc) return rc;
  if (!out) return AR_ERR_INVALID;
  if (!aligned16(out)) return AR_ERR_ALIGN;
  const Span so = span_of(out, n * 2);
  if ((rc = check_outputs(si, P, &so, 1))) return rc;
  if (n == 0) return AR_OK;
  ar::Launch L;
  if ((rc = resolve(&L, stream))) return rc;
  return hip_status(ar::launch_oneshot(L, in, P, out, n));
}

int ar_reduce_2stage(const void* const* ins, void* const* outs, int P, size_t n, void* scratch,
                     void* stream) {
  ar::InPtrs in{};
  ar::OutPtrs out{};
  Span si[AR_MAX_RANKS], so[AR_MAX_RANKS];
  int rc = check_ranks(ins, P, n, &in, si);
  if (rc) return rc;
  if (!outs) return AR_ERR_INVALID;
  for (int p = 0; p < P; ++p) {
    if (!outs[p]) return AR_ERR_INVALID;
    if (!aligned16(outs[p])) return AR_ERR_ALIGN;
    out.p[p] = outs[p];
    so[p] = span_of(outs[p], n * 2);
  }
  if ((rc = check_outputs(si, P, so, P))) return rc;
  if (scratch) {
    if (!aligned16(scratch)) return AR_ERR_ALIGN;
    const Span ss = span_of(scratch, n * 2);
    if ((rc = check_disjoint(ss, si, P)) || (rc = check_disjoint(ss, so, P))) return rc;
  }
  if (n == 0) return AR_OK;
  ar::Launch L;
  if ((rc = resolve(&L, stream))) return rc;
  if (scratch) return hip_status(ar::launch_2stage_staged(L, in, out, P, n, scratch));
  return hip_status(ar::launch_2stage_fused(L, in, out, P, n));
}

int ar_reduce_2stage_static(const void* const* ins, void* const* outs, int P, size_t n, void* stream) {
  ar::InPtrs in{};
  ar::OutPtrs out{};
  Span si[AR_MAX_RANKS], so[AR_MAX_RANKS];
  int rc = check_ranks(ins, P, n, &in, si);
  if (rc) return rc;
  if (!outs) return AR_ERR_INVALID;
  for (int p = 0; p < P; ++p) {
    if (!outs[p]) return AR_ERR_INVALID;
    if (!aligned16(outs[p])) return AR_ERR_ALIGN;
    out.p[p] = outs[p];
    so[p] = span_of(outs[p], n * 2);
  }
  if ((rc = check_outputs(si, P, so, P))) return rc;
  if (n > (size_t)AR_STATIC_SCRATCH_ELEMS) return AR_ERR_SIZE;
  if (n == 0) return AR_OK;
  ar::Launch L;
  if ((rc = resolve(&L, stream))) return rc;
  if (!L.scratch) return AR_ERR_HIP;
  return hip_status(ar::launch_2stage_staged(L, in, out, P, n, L.scratch));
}

int ar_pack_fused(const void* x, uint64_t* words, size_t n, uint32_t seq, void* stream) {
  if (!x || !words || (n & 1u) || mul_overflows(n, 4)) return AR_ERR_INVALID;
  if (!aligned16(x) || !aligned16(words)) return AR_ERR_ALIGN;
  if (overlap(span_of(x, n * 2), span_of(words, n * 4))) return AR_ERR_ALIAS;
  if (n == 0) return AR_OK;
  ar::Launch L;
  int rc = resolve(&L, stream);
  if (rc) return rc;
  return hip_status(ar::launch_pack(L, x, words, n, seq));
}

int ar_unpack_fused(const uint64_t* words, void* x, size_t n, uint32_t expected_seq, uint64_t* d_err,
                    void* stream) {
  if (!x || !words || (n & 1u) || mul_overflows(n, 4)) return AR_ERR_INVALID;
  int rc = check_err(d_err);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(words)) return AR_ERR_ALIGN;
  const Span sx = span_of(x, n * 2), sw = span_of(words, n * 4), se = span_of(d_err, 16);
  if (overlap(sx, sw) || overlap(se, sx) || overlap(se, sw)) return AR_ERR_ALIAS;
  if (n == 0) return AR_OK;
  ar::Launch L;
  if ((rc = resolve(&L, stream))) return rc;
  return hip_status(ar::launch_unpack(L, words, x, n, expected_seq, d_err));
}

int ar_unpack_fused_wait(const uint64_t* words, void* x, size_t n, uint32_t expected_seq,
                         uint32_t max_spins, uint64_t* d_err, void* stream) {
  if (!x || !words || (n & 1u) || mul_overflows(n, 4) || max_spins == 0) return AR_ERR_INVALID;
  int rc = check_err(d_err);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(words)) return AR_ERR_ALIGN;
  const Span sx = span_of(x, n * 2), sw = span_of(words, n * 4), se = span_of(d_err, 16);
  if (overlap(sx, sw) || overlap(se, sx) || overlap(se, sw)) return AR_ERR_ALIAS;
  if (n == 0) return AR_OK;
  ar::Launch L;
  if ((rc = resolve(&L, stream))) return rc;
  return hip_status(ar::launch_unpack_wait(L, words, x, n, expected_seq, max_spins, d_err));
}

int ar_quantize_fp8(const void* const* xs, uint8_t* const* codes, uint8_t* const* scales, int P,
                    size_t n, void* stream) {
  ar::InPtrs in{};
  ar::ByteOut co{}, sc{};
  Span si[AR_MAX_RANKS], sb[2 * AR_MAX_RANKS];
  int rc = check_ranks(xs, P, n, &in, si);
  if (rc) return rc;
  if (!codes || !scales) return AR_ERR_INVALID;
  const size_t nblk = (n + 31) / 32;
  for (int p = 0; p < P; ++p) {
    if (!codes[p] || !scales[p]) return AR_ERR_INVALID;
    if (!aligned16(codes[p])) return AR_ERR_ALIGN;
    co.p[p] = codes[p];
    sc.p[p] = scales[p];
    sb[2 * p] = span_of(codes[p], n);
    sb[2 * p + 1] = span_of(scales[p], nblk);
  }
  for (int a = 0; a < 2 * P; ++a) {
    if ((rc = check_disjoint(sb[a], si, P))) return rc;
    for (int b = a + 1; b < 2 * P; ++b)
      if (overlap(sb[a], sb[b])) return AR_ERR_ALIAS;
  }
  if (n == 0) return AR_OK;
  ar::Launch L;
  if ((rc = resolve(&L, stream))) return rc;
  return hip_status(ar::launch_quant_fp8(L, in, co, sc, P, n));
}

int ar_reduce_fp8(const uint8_t* const* codes, const uint8_t* const* scales, int P, void* const* outs,
                  int n_out, size_t n, void* stream) {
  if (!codes || !scales || !outs || P < 1 || P > AR_MAX_RANKS || mul_overflows(n, 2))
    return AR_ERR_INVALID;
  if (n_out != 1 && n_out != P) return AR_ERR_INVALID;
  ar::ByteIn co{}, sc{};
  ar::OutPtrs out{};
  Span sb[2 * AR_MAX_RANKS], so[AR_MAX_RANKS];
  const size_t nblk = (n + 31) / 32;
  for (int p = 0; p < P; ++p) {
    if (!codes[p] || !scales[p]) return AR_ERR_INVALID;
    if (!aligned16(codes[p])) return AR_ERR_ALIGN;
    co.p[p] = codes[p];
    sc.p[p] = scales[p];
    sb[2 * p] = span_of(codes[p], n);
    sb[2 * p + 1] = span_of(scales[p], nblk);
  }
  for (int o = 0; o < n_out; ++o) {
    if (!outs[o]) return AR_ERR_INVALID;
    if (!aligned16(outs[o])) return AR_ERR_ALIGN;
    out.p[o] = outs[o];
    so[o] = span_of(outs[o], n * 2);
  }
  int rc;
  if ((rc = check_outputs(so, 0, so, n_out))) return rc;
  for (int o = 0; o < n_out; ++o)
    if ((rc = check_disjoint(so[o], sb, 2 * P))) return rc;
  if (n == 0) return AR_OK;
  ar::Launch L;
  if ((rc = resolve(&L, stream))) return rc;
  return hip_status(ar::launch_reduce_fp8(L, co, sc, out, P, n_out, n));
}

int ar_rd_schedule(const uint64_t* const* in_words, uint64_t* const* out_words, int P, size_t n,
                   uint32_t seq0, uint64_t* mailbox, int flags, uint64_t* d_err, void* stream) {
  if (!in_words || !out_words || (n & 1u) || mul_overflows(n, 4)) return AR_ERR_INVALID;
  if (flags & ~(AR_RD_STAGED | AR_RD_FP32_CARRY)) return AR_ERR_INVALID;
  if (P != 2 && P != 4 && P != 8) return AR_ERR_UNSUPPORTED;
  const bool staged = (flags & AR_RD_STAGED) != 0;
  if (staged && (flags & AR_RD_FP32_CARRY)) return AR_ERR_UNSUPPORTED;
  int rc = check_err(d_err);
  if (rc) return rc;
  const int steps = P == 2 ? 1 : (P == 4 ? 2 : 3);
  ar::WordIn in{};
  ar::WordOut out{};
  Span si[AR_MAX_RANKS], so[AR_MAX_RANKS];
  for (int p = 0; p < P; ++p) {
    if (!in_words[p] || !out_words[p]) return AR_ERR_INVALID;
    if (!aligned16(in_words[p]) || !aligned16(out_words[p])) return AR_ERR_ALIGN;
    in.p[p] = in_words[p];
    out.p[p] = out_words[p];
    si[p] = span_of(in_words[p], n * 4);
    so[p] = span_of(out_words[p], n * 4);
  }
  if ((rc = check_outputs(si, P, so, P))) return rc;
  const Span se = span_of(d_err, 16);
  if ((rc = check_disjoint(se, si, P)) || (rc = check_disjoint(se, so, P))) return rc;
  if (staged && steps > 1) {
    if (!mailbox) return AR_ERR_INVALID;
    if (!aligned16(mailbox)) return AR_ERR_ALIGN;
    const size_t stride = ar::rd_mailbox_stride(n);
    if (mul_overflows((size_t)P * (size_t)(steps - 1), stride) ||
        mul_overflows((size_t)P * (size_t)(steps - 1) * stride, 8))
      return AR_ERR_INVALID;
    const size_t words = (size_t)P * (size_t)(steps - 1) * stride;
    const Span sm = span_of(mailbox, words * 8);
    if ((rc = check_disjoint(sm, si, P)) || (rc = check_disjoint(sm, so, P)) ||
        (rc = check_disjoint(sm, &se, 1)))
      return rc;
  }
  if (n == 0) return AR_OK;
  ar::Launch L;
  if ((rc = resolve(&L, stream))) return rc;
  if (staged) return hip_status(ar::launch_rd_staged(L, in, out, P, n, seq0, mailbox, d_err));
  return hip_status(
      ar::launch_rd_fused(L, in, out, P, n, seq0, (flags & AR_RD_FP32_CARRY) ? 1 : 0, d_err));
}

}  // extern "C"

namespace {

// Shared body of ar_reduce_ubatch and ar_reduce_ubatch_flags (done == NULL:
// no completion flags).
int ubatch_impl(const void* const* ins, void* const* outs, int P, size_t rows, size_t hidden,
                int n_ubatch, const size_t* ubatch_rows, size_t chunk_bytes, int variant,
                void* const* streams, uint32_t* done, uint32_t* tiles, size_t n_flags, uint32_t epoch) {
  const bool bounded = (variant & AR_UBATCH_BOUNDED) != 0;
  variant &= ~AR_UBATCH_BOUNDED;
  if (variant != AR_VARIANT_ONESHOT && variant != AR_VARIANT_2STAGE) return AR_ERR_INVALID;
  if (bounded && done) return AR_ERR_UNSUPPORTED;
  if (n_ubatch < 1 || n_ubatch > kMaxUbatch || !streams) return AR_ERR_INVALID;
  if (chunk_bytes == 0 || (chunk_bytes & 15u)) return AR_ERR_INVALID;
  if (mul_overflows(rows, hidden)) return AR_ERR_INVALID;
  const size_t n = rows * hidden;
  ar::InPtrs in{};
  ar::OutPtrs out{};
  Span si[AR_MAX_RANKS], so[AR_MAX_RANKS];
  int rc = check_ranks(ins, P, n, &in, si);
  if (rc) return rc;
  if (!outs) return AR_ERR_INVALID;
  const int nout = variant == AR_VARIANT_2STAGE ? P : 1;
  for (int p = 0; p < nout; ++p) {
    if (!outs[p]) return AR_ERR_INVALID;
    if (!aligned16(outs[p])) return AR_ERR_ALIGN;
    out.p[p] = outs[p];
    so[p] = span_of(outs[p], n * 2);
  }
  if ((rc = check_outputs(si, P, so, nout))) return rc;
  size_t split[kMaxUbatch];
  size_t total = 0;
  for (int u = 0; u < n_ubatch; ++u) {
    if (ubatch_rows) split[u] = ubatch_rows[u];
    else split[u] = (u == n_ubatch - 1) ? rows - total : rows / (size_t)n_ubatch;
    if (split[u] > rows - total) return AR_ERR_INVALID;
    total += split[u];
  }
  if (total != rows) return AR_ERR_INVALID;
  const size_t chunk = chunk_bytes / 2;
  if (done) {
    if (!tiles || epoch == 0) return AR_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(done) & 3u) || (reinterpret_cast<uintptr_t>(tiles) & 3u))
      return AR_ERR_ALIGN;
    size_t need = 0;
    for (int u = 0; u < n_ubatch; ++u) need += (split[u] * hidden + chunk - 1) / chunk;
    if (need > n_flags || need > 0xFFFFFFFFull || mul_overflows(n_flags, 4)) return AR_ERR_INVALID;
    const Span sd = span_of(done, n_flags * 4), st = span_of(tiles, n_flags * 4);
    if (overlap(sd, st) || check_disjoint(sd, si, P) || check_disjoint(sd, so, nout) ||
        check_disjoint(st, si, P) || check_disjoint(st, so, nout))
      return AR_ERR_ALIAS;
  }
  if (n == 0) return AR_OK;
  ar::Launch L;
  if ((rc = resolve(&L, nullptr))) return rc;
  // every ubatch's grid is checked before the first launch
  size_t row0 = 0, chunk0 = 0;
  for (int u = 0; u < n_ubatch; ++u) {
    const size_t e0 = row0 * hidden, e1 = (row0 + split[u]) * hidden;
    row0 += split[u];
    if (e1 > e0 && !ar::chunked_fits(L, e0, e1, chunk, nout > 1 ? 1 : 0, done != nullptr, bounded))
      return AR_ERR_INVALID;
  }
  row0 = 0;
  for (int u = 0; u < n_ubatch; ++u) {
    const size_t e0 = row0 * hidden, e1 = (row0 + split[u]) * hidden;
    row0 += split[u];
    if (e1 == e0) continue;
    L.stream = static_cast<hipStream_t>(streams[u]);
    const ar::ChunkSignal sig{done, done ? tiles : nullptr, epoch, (uint32_t)chunk0};
    rc = hip_status(bounded ? ar::launch_chunked_bounded(L, in, out, P, e0, e1, chunk, nout > 1 ? 1 : 0)
                            : ar::launch_chunked(L, in, out, P, e0, e1, chunk, nout > 1 ? 1 : 0, sig));
    if (rc) return rc;
    chunk0 += (e1 - e0 + chunk - 1) / chunk;
  }
  return AR_OK;
}

}  // namespace

extern "C" {

int ar_reduce_ubatch(const void* const* ins, void* const* outs, int P, size_t rows, size_t hidden,
                     int n_ubatch, const size_t* ubatch_rows, size_t chunk_bytes, int variant,
                     void* const* streams) {
  return ubatch_impl(ins, outs, P, rows, hidden, n_ubatch, ubatch_rows, chunk_bytes, variant, streams,
                     nullptr, nullptr, 0, 0);
}

int ar_reduce_ubatch_flags(const void* const* ins, void* const* outs, int P, size_t rows,
                           size_t hidden, int n_ubatch, const size_t* ubatch_rows, size_t chunk_bytes,
                           int variant, void* const* streams, uint32_t* chunk_done,
                           uint32_t* chunk_tiles, size_t n_flags, uint32_t epoch) {
  if (!chunk_done) return AR_ERR_INVALID;
  return ubatch_impl(ins, outs, P, rows, hidden, n_ubatch, ubatch_rows, chunk_bytes, variant, streams,
                     chunk_done, chunk_tiles, n_flags, epoch);
}

int ar_set_launch_shape(int kind, int block, int vec, int nt_loads, int stores, int wg_per_cu) {
  if (kind < 0 || kind >= ar::kKinds || !shape_ok(kind, block, vec, nt_loads, stores, wg_per_cu))
    return AR_ERR_INVALID;
  std::lock_guard<std::mutex> lock(g_mu);
  init_base_locked();
  g_base[kind] = ar::Shape{block, vec, nt_loads, stores, wg_per_cu, 0};
  // republish every device already in use; later calls see the new shape
  for (int d = 0; d < kMaxDevices; ++d)
    if (g_table[d].load(std::memory_order_relaxed)) publish_locked(d, false);
  return AR_OK;
}

int ar_get_launch_shape(int kind, int* block, int* vec, int* nt_loads, int* stores,
                        int* wg_per_cu) {
  if (kind < 0 || kind >= ar::kKinds || !block || !vec || !nt_loads || !stores || !wg_per_cu)
    return AR_ERR_INVALID;
  std::lock_guard<std::mutex> lock(g_mu);
  init_base_locked();
  const ar::Shape& s = g_base[kind];
  *block = s.block;
  *vec = s.vec;
  *nt_loads = s.nt_loads;
  *stores = s.stores;
  *wg_per_cu = s.wg_per_cu;
  return AR_OK;
}

int ar_err_init(uint64_t* d_err, void* stream) {
  int rc = check_err(d_err);
  if (rc) return rc;
  ar::Launch L;
  if ((rc = resolve(&L, stream))) return rc;
  return hip_status(ar::launch_err_init(L, d_err));
}

}  // extern "C"
