/*
 * CPU oracle of the multi-buffer all-reduce core.  TEST INFRASTRUCTURE ONLY:
 * nothing on the product path may include, link or call this file.  Only the
 * test suite, the smoke check and the bench's CPU-baseline leg use it.
 *
 * Plain, slow and literal on purpose: every function walks the schedule in
 * the order the pages describe, element by element, with no blocking, fusion
 * or reordering.  It shares no code, header or table with the HIP library.
 *
 * Pages cited (titles as printed):
 *   [TBO-AR]  "[DSV4] perf(tbo): overlap pure-TP all_reduce on TBO + Delay TP"
 *   [CAR]     "fix(custom_all_reduce): use SYSTEM scope + ACQUIRE ordering for
 *              cross-device signal loads"
 *   [NVRAR]   "Technical Summary: Understanding and Improving Communication
 *              Performance in Multi-node LLM Inference"
 *
 * Numerics (a reading; the pages only say the models run in bf16, [NVRAR]
 * Methodology 1 "Models"): every sum is taken in IEEE-754 binary32 with
 * round-to-nearest-even, subnormals kept, no fused multiply-add and no
 * reassociation, starting from rank 0's value and adding ranks 1..P-1 in
 * order; the binary32 result is rounded once to bf16 (nearest, ties to even),
 * any NaN result becomes the canonical quiet NaN 0x7FC0.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 *        -fexcess-precision=standard  (x86-64: SSE2 binary32 arithmetic)
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MAX_P 64

/* bf16 bits -> binary32 value.  bf16 is the top half of a binary32, so the
 * widening is exact: the 16 bf16 bits become the high 16 bits. */
float orc_widen(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 value -> bf16 bits, round to nearest, ties to even.
 * Keeping the high 16 bits truncates the magnitude; the low 16 discarded bits
 * decide: above half a bf16 ulp rounds the magnitude up, below rounds down,
 * exactly half rounds to the candidate whose last kept bit is 0.  A carry out
 * of the mantissa moves to the next binade, and past the largest finite value
 * gives infinity, as nearest rounding requires.  NaN -> 0x7FC0. */
uint16_t orc_rn(float a) {
    if (isnan(a)) return 0x7FC0u;
    uint32_t u;
    memcpy(&u, &a, sizeof u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

void orc_rn_array(const float* a, size_t n, uint16_t* out) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_rn(a[i]);
}

/* Sequential fixed-order sum of element i over P rank buffers:
 * acc = x_0[i]; acc = acc + x_p[i] for p = 1..P-1 (binary32); one rounding. */
static uint16_t seq_sum_at(int P, const uint16_t* const* xs, size_t i) {
    float acc = orc_widen(xs[0][i]);
    for (int p = 1; p < P; ++p) acc = acc + orc_widen(xs[p][i]);
    return orc_rn(acc);
}

/* One-shot reduce: one output holding the sum of all P buffers.
 * ([CAR] names only the two-stage kernel; a one-stage reduce, where a rank
 * reads every peer buffer and sums, is the plain reading of what two-stage
 * splits in two.) */
void orc_reduce_seq(int P, const uint16_t* const* xs, size_t n, uint16_t* out) {
    for (size_t i = 0; i < n; ++i) out[i] = seq_sum_at(P, xs, i);
}

/* Shard length of the two-stage reduce: each of the P shards covers
 * ceil(ceil(n/8)/P) groups of 8 elements, so every shard starts on a 16-byte
 * boundary; trailing shards may be short or empty. */
size_t orc_shard_len(int P, size_t n) {
    size_t groups = (n + 7) / 8;
    size_t per = (groups + (size_t)P - 1) / (size_t)P;
    return per * 8;
}

/* Two-stage reduce ([CAR] Changes 3 / Root cause: the 2-stage write-mode
 * kernel; [NVRAR] Methodology 3, phases 1 and 3).
 * Stage 1, reduce-scatter: the owner of shard s sums shard s over all P
 * buffers (same order as the one-shot) into scratch.
 * Stage 2, all-gather: every rank's output receives every reduced shard.
 * scratch may be NULL, in which case a private buffer is used. */
int orc_reduce_2stage(int P, const uint16_t* const* xs, size_t n,
                      uint16_t* scratch, uint16_t* const* outs) {
    uint16_t* red = scratch;
    if (red == NULL && n > 0) {
        red = (uint16_t*)malloc(n * sizeof *red);
        if (red == NULL) return -1;
    }
    size_t S = orc_shard_len(P, n);
    for (int s = 0; s < P; ++s) {                 /* stage 1 */
        size_t lo = (size_t)s * S;
        size_t hi = lo + S < n ? lo + S : n;
        for (size_t i = lo; i < hi; ++i) red[i] = seq_sum_at(P, xs, i);
    }
    for (int r = 0; r < P; ++r) {                 /* stage 2 */
        for (int s = 0; s < P; ++s) {
            size_t lo = (size_t)s * S;
            size_t hi = lo + S < n ? lo + S : n;
            for (size_t i = lo; i < hi; ++i) outs[r][i] = red[i];
        }
    }
    if (red != scratch) free(red);
    return 0;
}

/* Two-ubatch chunked reduce ([TBO-AR] pull request overview: each ubatch's TP
 * all-reduce runs on its own stream; [NVRAR] Optimizations, "Chunked
 * Non-blocking Communication").  Rows are split into ubatches (ub_rows NULL:
 * even split, remainder to the last); each ubatch walks its element range in
 * ascending chunks of chunk_elems elements of every rank buffer.
 * variant 0 = one-shot (outs[0] only), 1 = two-stage (all P outputs). */
int orc_reduce_ubatch(int P, const uint16_t* const* xs, uint16_t* const* outs,
                      size_t rows, size_t hidden, int n_ub,
                      const size_t* ub_rows, size_t chunk_elems, int variant) {
    if (n_ub < 1 || chunk_elems == 0) return -1;
    size_t row0 = 0;
    for (int u = 0; u < n_ub; ++u) {
        size_t ur;
        if (ub_rows != NULL) ur = ub_rows[u];
        else ur = (u == n_ub - 1) ? rows - row0 : rows / (size_t)n_ub;
        size_t e0 = row0 * hidden, e1 = (row0 + ur) * hidden;
        for (size_t c0 = e0; c0 < e1; c0 += chunk_elems) {
            size_t c1 = c0 + chunk_elems < e1 ? c0 + chunk_elems : e1;
            for (size_t i = c0; i < c1; ++i) {
                uint16_t v = seq_sum_at(P, xs, i);
                if (variant == 0) outs[0][i] = v;
                else for (int r = 0; r < P; ++r) outs[r][i] = v;
            }
        }
        row0 += ur;
    }
    return row0 == rows ? 0 : -1;
}

/* Fused 8-byte payload ([NVRAR] Optimizations, "Fused Payloads": data and the
 * synchronisation flag travel in one 8-byte word).  Layout (a reading; the
 * page gives none): bits 0-15 element 2j, bits 16-31 element 2j+1, bits
 * 32-63 the sequence number. */
static uint64_t make_word(uint16_t lo, uint16_t hi, uint32_t seq) {
    return ((uint64_t)seq << 32) | ((uint64_t)hi << 16) | (uint64_t)lo;
}

void orc_pack(const uint16_t* x, size_t n, uint32_t seq, uint64_t* w) {
    for (size_t j = 0; j < n / 2; ++j) w[j] = make_word(x[2 * j], x[2 * j + 1], seq);
}

/* Unpack and check ([NVRAR] Optimizations, "Sequence-Number
 * Synchronization": a unique sequence number marks a payload as current).
 * Data is written whatever the check says; err[0] += number of words whose
 * sequence number differs, err[1] = min(err[1], index of the first such word). */
void orc_unpack(const uint64_t* w, size_t n, uint32_t expected, uint16_t* x,
                uint64_t* err) {
    for (size_t j = 0; j < n / 2; ++j) {
        x[2 * j] = (uint16_t)(w[j] & 0xFFFFu);
        x[2 * j + 1] = (uint16_t)((w[j] >> 16) & 0xFFFFu);
        if ((uint32_t)(w[j] >> 32) != expected) {
            err[0] += 1;
            if ((uint64_t)j < err[1]) err[1] = (uint64_t)j;
        }
    }
}

/* Recursive doubling over P = 2^L simulated ranks ([NVRAR] Methodology 3,
 * phase 2 "Inter-node Recursive-Doubling"; Optimizations "Fused Payloads",
 * "Sequence-Number Synchronization").
 * Step k = 0..L-1: rank r exchanges with partner q = r XOR 2^k.  Every rank
 * receives its partner's payload, checks that it carries seq0 + k, and
 * combines.  fp32_carry == 0 (default): the exchanged partial is the bf16
 * payload, so each combine is rn(f(own) + f(partner)) and the new payload
 * carries seq0 + k + 1.  fp32_carry == 1: partials stay binary32 between
 * steps and are rounded once at the end (no payload between steps).
 * Output payloads carry seq0 + L.  err[0] counts received words with a wrong
 * sequence number; err[1] = min over them of (k*P + q)*W + j, where q is the
 * rank whose payload was received and W = n/2. */
int orc_rd(int P, const uint64_t* const* in, size_t n, uint32_t seq0,
           int fp32_carry, uint64_t* const* out, uint64_t* err) {
    int L = 0;
    while ((1 << L) < P) ++L;
    if (P < 2 || P > ORC_MAX_P || (1 << L) != P || (n & 1u)) return -1;
    size_t W = n / 2;
    /* state[r][2j], state[r][2j+1]: rank r's current partial of elements 2j, 2j+1 */
    float* cur = (float*)malloc((size_t)P * n * sizeof(float));
    float* nxt = (float*)malloc((size_t)P * n * sizeof(float));
    uint32_t* seq = (uint32_t*)malloc((size_t)P * W * sizeof(uint32_t));
    if (!cur || !nxt || !seq) { free(cur); free(nxt); free(seq); return -1; }
    for (int r = 0; r < P; ++r)
        for (size_t j = 0; j < W; ++j) {
            cur[(size_t)r * n + 2 * j] = orc_widen((uint16_t)(in[r][j] & 0xFFFFu));
            cur[(size_t)r * n + 2 * j + 1] = orc_widen((uint16_t)((in[r][j] >> 16) & 0xFFFFu));
            seq[(size_t)r * W + j] = (uint32_t)(in[r][j] >> 32);
        }
    for (int k = 0; k < L; ++k) {
        uint32_t want = seq0 + (uint32_t)k;
        for (int r = 0; r < P; ++r) {
            int q = r ^ (1 << k);
            for (size_t j = 0; j < W; ++j) {
                if (seq[(size_t)q * W + j] != want) {
                    uint64_t idx = ((uint64_t)k * (uint64_t)P + (uint64_t)q) * W + j;
                    err[0] += 1;
                    if (idx < err[1]) err[1] = idx;
                }
                for (int h = 0; h < 2; ++h) {
                    float a = cur[(size_t)r * n + 2 * j + h];
                    float b = cur[(size_t)q * n + 2 * j + h];
                    float s = a + b;
                    nxt[(size_t)r * n + 2 * j + h] = fp32_carry ? s : orc_widen(orc_rn(s));
                }
            }
        }
        /* every rank now holds the step-(k+1) payload */
        for (size_t t = 0; t < (size_t)P * W; ++t) seq[t] = seq0 + (uint32_t)k + 1u;
        float* tmp = cur; cur = nxt; nxt = tmp;
    }
    for (int r = 0; r < P; ++r)
        for (size_t j = 0; j < W; ++j)
            out[r][j] = make_word(orc_rn(cur[(size_t)r * n + 2 * j]),
                                  orc_rn(cur[(size_t)r * n + 2 * j + 1]),
                                  seq0 + (uint32_t)L);
    free(cur); free(nxt); free(seq);
    return 0;
}

/* ---------------------------------------------------------------------------
 * fp8-quantised contributions ([TBO-AR] diff, the caller passes the
 * ca_fp8_quant flag of the custom all-reduce; the pages give no scheme).
 * Reading taken here: each rank's bf16 contribution travels as fp8 E4M3
 * codes (the OCP "FN" variant: bias 7, no infinities, 0x7F/0xFF are NaN,
 * largest finite 448) with one power-of-two scale per block of 32
 * consecutive elements, the block/scale layout of the OCP Microscaling
 * formats; the scale is the smallest power of two at which no element of
 * the block exceeds 448 (so nothing clips).  The receiver dequantises
 * exactly (code value times the scale) and sums in binary32 in rank order
 * 0..P-1, then rounds once to bf16 as orc_reduce_seq does.
 * ------------------------------------------------------------------------- */

#define ORC_FP8_BLOCK 32

/* Value of an E4M3 code: sign bit 7, exponent bits 6..3 (bias 7), mantissa
 * bits 2..0.  Exponent 0: subnormal m * 2^-9; otherwise (1 + m/8) * 2^(e-7);
 * exponent 15 with mantissa 7 is NaN. */
float orc_e4m3_value(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (float)(s ? -v : v);
}

/* Nearest E4M3 code to v, ties to the code with an even mantissa.  Defined
 * for |v| <= 448; a larger or non-finite v gives the NaN code 0x7F.  The
 * non-negative codes 0x00..0x7E are in increasing order of value, so the
 * candidates are the largest code not above |v| and the next one.  The sign
 * is kept, so a negative value that rounds to zero gives 0x80. */
uint8_t orc_e4m3_rn(double v) {
    if (!(fabs(v) <= 448.0)) return 0x7Fu;
    double a = fabs(v);
    uint8_t lo = 0;
    while (lo < 0x7E && (double)orc_e4m3_value((uint8_t)(lo + 1)) <= a) ++lo;
    uint8_t c = lo;
    if (lo < 0x7E) {
        double dl = a - (double)orc_e4m3_value(lo);
        double dh = (double)orc_e4m3_value((uint8_t)(lo + 1)) - a;
        if (dh < dl || (dh == dl && (lo & 1u))) c = (uint8_t)(lo + 1);
    }
    return (uint8_t)((signbit(v) ? 0x80u : 0u) | c);
}

void orc_e4m3_rn_array(const double* v, size_t n, uint8_t* out) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_e4m3_rn(v[i]);
}

/* Scale exponent of one block: the smallest k in [-127, 127] with
 * amax <= 448 * 2^k, amax = the largest |x| over the block's finite
 * elements (0 if none). */
int orc_fp8_block_exp(const uint16_t* x, size_t len) {
    double amax = 0.0;
    for (size_t i = 0; i < len; ++i) {
        double f = (double)orc_widen(x[i]);
        if (isfinite(f) && fabs(f) > amax) amax = fabs(f);
    }
    int k = -127;
    while (k < 127 && amax > ldexp(448.0, k)) ++k;
    return k;
}

/* Quantise one rank buffer of n bf16 elements: scales[b] = k_b + 127 for
 * block b (ceil(n/32) blocks, the last one possibly short), and
 * codes[i] = rn_e4m3(x_i / 2^k_b); a NaN or infinite x_i gives 0x7F. */
void orc_quant_fp8(const uint16_t* x, size_t n, uint8_t* codes, uint8_t* scales) {
    for (size_t b0 = 0; b0 < n; b0 += ORC_FP8_BLOCK) {
        size_t len = n - b0 < ORC_FP8_BLOCK ? n - b0 : ORC_FP8_BLOCK;
        int k = orc_fp8_block_exp(x + b0, len);
        scales[b0 / ORC_FP8_BLOCK] = (uint8_t)(k + 127);
        for (size_t i = b0; i < b0 + len; ++i) {
            double f = (double)orc_widen(x[i]);
            codes[i] = isfinite(f) ? orc_e4m3_rn(ldexp(f, -k)) : (uint8_t)0x7Fu;
        }
    }
}

/* Dequantised value of element i of one rank: code value times 2^k, exact
 * in binary32 except at the top of the range: a block whose maximum is
 * 1.9375 * 2^127 or more (the 8 largest finite bf16 magnitudes) gets k = 120
 * and that element the code of 256, and 256 * 2^120 = 2^128 is infinite in
 * binary32, as rounding such a value to bf16 directly would also be. */
float orc_dequant_fp8(const uint8_t* codes, const uint8_t* scales, size_t i) {
    int k = (int)scales[i / ORC_FP8_BLOCK] - 127;
    return (float)ldexp((double)orc_e4m3_value(codes[i]), k);
}

/* out[i] = rn(((d_0 + d_1) + d_2) + ... + d_{P-1}) over the dequantised
 * contributions, binary32 sums in rank order, one bf16 rounding. */
int orc_reduce_fp8(int P, const uint8_t* const* codes, const uint8_t* const* scales, size_t n,
                   uint16_t* out) {
    if (P < 1 || P > ORC_MAX_P) return -1;
    for (size_t i = 0; i < n; ++i) {
        float acc = orc_dequant_fp8(codes[0], scales[0], i);
        for (int p = 1; p < P; ++p) acc = acc + orc_dequant_fp8(codes[p], scales[p], i);
        out[i] = orc_rn(acc);
    }
    return 0;
}

int orc_version(void) { return 1; }
