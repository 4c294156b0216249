/*
 * The C-ABI used from plain C (C99, no Python, no torch): device buffers
 * from the HIP C API, every main entry point of ar.h called on one stream,
 * results copied back and checked.
 *
 * Inputs are small integers (rank p, element i: ((7 i + 13 p) mod 33) - 16,
 * in [-16, 16]), so every partial sum over P = 8 ranks is an integer of
 * magnitude at most 128: exact in binary32 and in bf16 whatever the order of
 * the additions.  Every schedule (one-shot, both two-stage modes, the fused
 * one in place, the staged one on the static scratch, recursive doubling
 * with bf16 or binary32 partials, the two-stream ubatch reduce)
 * must therefore return exactly the integer sum, which this program computes
 * on its own with integer arithmetic.  n is ragged (not a multiple of 8) and
 * spans many tiles.
 *
 * c_abi_check() returns 0 when every check passes, 1 at the first mismatch
 * and 2 on a HIP or library error; c_abi_check_message() then describes the
 * outcome in one line.  The tests load this file built as a shared object
 * and call it in their own process; built with -DC_ABI_CHECK_MAIN it is a
 * program of its own that prints the line.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ar.h"

static char g_msg[512];

/* One line describing the last c_abi_check() outcome. */
const char* c_abi_check_message(void) { return g_msg; }

#define P 8
#define ROWS 9
#define HIDDEN 8190
#define N ((size_t)ROWS * HIDDEN) /* 73710 elements: even, not a multiple of 8 */

#define HIP(call)                                                                          \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) {                                                                \
      snprintf(g_msg, sizeof g_msg, "c-abi check: %s failed: %s", #call,                   \
               hipGetErrorString(e_));                                                     \
      return 2;                                                                            \
    }                                                                                      \
  } while (0)

#define AR(call)                                                                           \
  do {                                                                                     \
    int r_ = (call);                                                                       \
    if (r_ != AR_OK) {                                                                     \
      snprintf(g_msg, sizeof g_msg, "c-abi check: %s returned %s", #call, ar_status_str(r_)); \
      return 2;                                                                            \
    }                                                                                      \
  } while (0)

/* bf16 bit pattern of a small integer v (|v| <= 256): exact. */
static uint16_t bf16_of_int(int v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static int value(size_t i, int p) { return (int)((7 * i + 13 * (size_t)p) % 33) - 16; }

static int check16(const char* what, const uint16_t* got, const uint16_t* want, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    if (got[i] != want[i]) {
      snprintf(g_msg, sizeof g_msg, "c-abi check: %s differs at %zu: got 0x%04X want 0x%04X", what, i,
               got[i], want[i]);
      return 1;
    }
  }
  return 0;
}

int c_abi_check(void) {
  uint16_t* host[P];
  uint16_t* want = malloc(N * 2);
  uint16_t* got = malloc(N * 2);
  if (!want || !got) return 2;
  for (int p = 0; p < P; ++p) {
    host[p] = malloc(N * 2);
    if (!host[p]) return 2;
  }
  for (size_t i = 0; i < N; ++i) {
    int s = 0;
    for (int p = 0; p < P; ++p) {
      host[p][i] = bf16_of_int(value(i, p));
      s += value(i, p);
    }
    want[i] = bf16_of_int(s);
  }

  hipStream_t st, st2;
  HIP(hipStreamCreate(&st));
  HIP(hipStreamCreate(&st2));
  void *ins[P], *outs[P], *out1, *scratch, *x;
  uint64_t *words[P], *rdo[P], *mbox, *err;
  for (int p = 0; p < P; ++p) {
    HIP(hipMalloc(&ins[p], N * 2));
    HIP(hipMalloc(&outs[p], N * 2));
    HIP(hipMalloc((void**)&words[p], N * 4));
    HIP(hipMalloc((void**)&rdo[p], N * 4));
    HIP(hipMemcpy(ins[p], host[p], N * 2, hipMemcpyHostToDevice));
  }
  HIP(hipMalloc(&out1, N * 2));
  HIP(hipMalloc(&scratch, N * 2));
  HIP(hipMalloc(&x, N * 2));
  /* mailbox: P * (log2 P - 1) payloads of W words, W rounded up to even */
  const size_t W = N / 2, Ws = W + (W & 1);
  HIP(hipMalloc((void**)&mbox, (size_t)P * 2 * Ws * 8));
  HIP(hipMalloc((void**)&err, 16));

  int bad = 0;
  /* one-shot */
  AR(ar_reduce_oneshot((const void* const*)ins, P, out1, N, st));
  HIP(hipStreamSynchronize(st));
  HIP(hipMemcpy(got, out1, N * 2, hipMemcpyDeviceToHost));
  bad |= check16("one-shot", got, want, N);

  /* two-stage, fused then staged */
  for (int staged = 0; staged < 2 && !bad; ++staged) {
    for (int p = 0; p < P; ++p) HIP(hipMemset(outs[p], 0, N * 2));
    AR(ar_reduce_2stage((const void* const*)ins, outs, P, N, staged ? scratch : NULL, st));
    HIP(hipStreamSynchronize(st));
    for (int p = 0; p < P && !bad; ++p) {
      HIP(hipMemcpy(got, outs[p], N * 2, hipMemcpyDeviceToHost));
      bad |= check16(staged ? "staged two-stage" : "fused two-stage", got, want, N);
    }
  }

  /* fused two-stage in place (each rank's result in its own buffer), then the
     staged two-stage on the library's static scratch */
  if (!bad) {
    for (int p = 0; p < P; ++p) HIP(hipMemcpy(outs[p], ins[p], N * 2, hipMemcpyDeviceToDevice));
    AR(ar_reduce_2stage((const void* const*)outs, outs, P, N, NULL, st));
    HIP(hipStreamSynchronize(st));
    for (int p = 0; p < P && !bad; ++p) {
      HIP(hipMemcpy(got, outs[p], N * 2, hipMemcpyDeviceToHost));
      bad |= check16("in-place two-stage", got, want, N);
    }
  }
  if (!bad) {
    for (int p = 0; p < P; ++p) HIP(hipMemset(outs[p], 0, N * 2));
    AR(ar_reduce_2stage_static((const void* const*)ins, outs, P, N, st));
    HIP(hipStreamSynchronize(st));
    for (int p = 0; p < P && !bad; ++p) {
      HIP(hipMemcpy(got, outs[p], N * 2, hipMemcpyDeviceToHost));
      bad |= check16("static-scratch two-stage", got, want, N);
    }
  }

  /* pack -> recursive doubling (fused R1, fused R2, staged) -> unpack */
  const int modes[3] = {0, AR_RD_FP32_CARRY, AR_RD_STAGED};
  for (int k = 0; k < 3 && !bad; ++k) {
    const uint32_t seq0 = 0xFFFFFFFEu; /* wraps during the call */
    AR(ar_err_init(err, st));
    for (int p = 0; p < P; ++p) AR(ar_pack_fused(ins[p], words[p], N, seq0, st));
    AR(ar_rd_schedule((const uint64_t* const*)words, rdo, P, N, seq0, k == 2 ? mbox : NULL, modes[k], err,
                      st));
    for (int p = 0; p < P && !bad; ++p) {
      HIP(hipMemset(x, 0, N * 2));
      AR(ar_unpack_fused(rdo[p], x, N, seq0 + 3u, err, st));
      HIP(hipStreamSynchronize(st));
      HIP(hipMemcpy(got, x, N * 2, hipMemcpyDeviceToHost));
      bad |= check16("pack, recursive doubling, unpack", got, want, N);
    }
    uint64_t e[2];
    HIP(hipMemcpy(e, err, 16, hipMemcpyDeviceToHost));
    if (!bad && (e[0] != 0 || e[1] != ~(uint64_t)0)) {
      snprintf(g_msg, sizeof g_msg, "c-abi check: recursive doubling mode %d counted %llu stale words", k,
               (unsigned long long)e[0]);
      bad = 1;
    }
  }

  /* two-ubatch reduce on two streams, chunks not aligned to rows */
  if (!bad) {
    for (int p = 0; p < P; ++p) HIP(hipMemset(outs[p], 0, N * 2));
    HIP(hipDeviceSynchronize());
    void* streams[2] = {st, st2};
    AR(ar_reduce_ubatch((const void* const*)ins, outs, P, ROWS, HIDDEN, 2, NULL, 4096 + 16, AR_VARIANT_2STAGE,
                        streams));
    HIP(hipDeviceSynchronize());
    for (int p = 0; p < P && !bad; ++p) {
      HIP(hipMemcpy(got, outs[p], N * 2, hipMemcpyDeviceToHost));
      bad |= check16("two-stream ubatch", got, want, N);
    }
  }

  /* argument errors are returned before any work */
  if (!bad && ar_reduce_oneshot((const void* const*)ins, P, (char*)out1 + 2, N, st) != AR_ERR_ALIGN) {
    snprintf(g_msg, sizeof g_msg, "c-abi check: a misaligned output was not refused");
    bad = 1;
  }

  for (int p = 0; p < P; ++p) {
    (void)hipFree(ins[p]);
    (void)hipFree(outs[p]);
    (void)hipFree(words[p]);
    (void)hipFree(rdo[p]);
    free(host[p]);
  }
  (void)hipFree(out1);
  (void)hipFree(scratch);
  (void)hipFree(x);
  (void)hipFree(mbox);
  (void)hipFree(err);
  (void)hipStreamDestroy(st);
  (void)hipStreamDestroy(st2);
  free(want);
  free(got);
  if (bad) return 1;
  snprintf(g_msg, sizeof g_msg,
           "c-abi check: one-shot, two-stage (fused, staged, in place, static scratch), recursive doubling "
           "(R1, R2, staged) and the two-stream ubatch reduce exact on %d x %zu elements (library version %d)",
           P, N, ar_version());
  return 0;
}

#ifdef C_ABI_CHECK_MAIN
int main(void) {
  const int rc = c_abi_check();
  puts(c_abi_check_message());
  return rc;
}
#endif
