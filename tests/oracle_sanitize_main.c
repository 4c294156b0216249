/*
 * Memory-safety driver for the oracle (test infrastructure): compiled
 * together with oracle/ar_oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_oracle_sanitize.py, it calls every
 * oracle function on edge-case sizes -- empty, one element, ragged tails,
 * odd word counts, short fp8 blocks -- with every buffer allocated to its
 * exact length, so any read or write past an end, use of freed memory or
 * undefined arithmetic aborts the run.  Values are not checked here (the
 * pins do that); the run must finish with exit status 0 and no report.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../oracle/ar_oracle.c"

static uint32_t lcg = 12345u;
static uint16_t rnd16(void) {
    lcg = lcg * 1664525u + 1013904223u;
    return (uint16_t)(lcg >> 16);
}

static uint16_t* bufs16(int P, size_t n, uint16_t** v) {
    for (int p = 0; p < P; ++p) {
        v[p] = (uint16_t*)malloc(n ? n * 2 : 1);
        for (size_t i = 0; i < n; ++i) v[p][i] = rnd16();
    }
    return v[0];
}

static void free_all(int P, void** v) {
    for (int p = 0; p < P; ++p) free(v[p]);
}

int main(void) {
    static const size_t sizes[] = {0, 1, 2, 3, 7, 8, 9, 31, 32, 33, 64, 65, 1000, 4098};
    static const int Ps[] = {1, 2, 3, 4, 8};
    for (size_t si = 0; si < sizeof sizes / sizeof *sizes; ++si) {
        const size_t n = sizes[si];
        for (size_t pi = 0; pi < sizeof Ps / sizeof *Ps; ++pi) {
            const int P = Ps[pi];
            uint16_t* xs[8];
            uint16_t* outs[8];
            bufs16(P, n, xs);
            bufs16(P, n, outs);
            uint16_t* one = (uint16_t*)malloc(n ? n * 2 : 1);
            orc_reduce_seq(P, (const uint16_t* const*)xs, n, one);
            uint16_t* scratch = (uint16_t*)malloc(n ? n * 2 : 1);
            if (orc_reduce_2stage(P, (const uint16_t* const*)xs, n, scratch, outs)) return 2;
            if (orc_reduce_2stage(P, (const uint16_t* const*)xs, n, NULL, outs)) return 3;
            /* ubatch: rows x hidden = n for the sizes that split */
            if (n % 8 == 0 && n > 0) {
                const size_t rows = 8, hidden = n / 8;
                const size_t split[3] = {3, 0, 5};
                if (orc_reduce_ubatch(P, (const uint16_t* const*)xs, outs, rows, hidden, 3, split, 5, 1)) return 4;
                if (orc_reduce_ubatch(P, (const uint16_t* const*)xs, outs, rows, hidden, 2, NULL, 16, 0)) return 5;
            }
            /* fused payloads (even n) and recursive doubling (P a power of two) */
            if (n % 2 == 0) {
                uint64_t* w[8];
                uint64_t* wo[8];
                for (int p = 0; p < P; ++p) {
                    w[p] = (uint64_t*)malloc(n ? n * 4 : 1);
                    wo[p] = (uint64_t*)malloc(n ? n * 4 : 1);
                    orc_pack(xs[p], n, 0xFFFFFFFFu, w[p]);
                }
                uint64_t err[2] = {0, ~0ull};
                orc_unpack(w[0], n, 0xFFFFFFFFu, one, err);
                if (P == 2 || P == 4 || P == 8) {
                    if (orc_rd(P, (const uint64_t* const*)w, n, 0xFFFFFFFEu, 0, wo, err)) return 6;
                    if (orc_rd(P, (const uint64_t* const*)w, n, 7u, 1, wo, err)) return 7;
                }
                free_all(P, (void**)w);
                free_all(P, (void**)wo);
            }
            /* fp8 contributions: codes n bytes, scales ceil(n/32) bytes, exactly */
            uint8_t* codes[8];
            uint8_t* scales[8];
            const size_t nb = (n + 31) / 32;
            for (int p = 0; p < P; ++p) {
                codes[p] = (uint8_t*)malloc(n ? n : 1);
                scales[p] = (uint8_t*)malloc(nb ? nb : 1);
                orc_quant_fp8(xs[p], n, codes[p], scales[p]);
            }
            if (orc_reduce_fp8(P, (const uint8_t* const*)codes, (const uint8_t* const*)scales, n, one)) return 8;
            free_all(P, (void**)codes);
            free_all(P, (void**)scales);
            free_all(P, (void**)xs);
            free_all(P, (void**)outs);
            free(one);
            free(scratch);
        }
    }
    /* scalar helpers over their whole domains */
    for (uint32_t c = 0; c < 256; ++c) (void)orc_e4m3_value((uint8_t)c);
    for (int i = -2000; i <= 2000; ++i) (void)orc_e4m3_rn(i * 0.25);
    for (uint32_t b = 0; b < 65536; ++b) (void)orc_rn(orc_widen((uint16_t)b));
    (void)orc_shard_len(8, 0);
    (void)orc_shard_len(3, 1001);
    printf("oracle sanitize run: ok\n");
    return 0;
}
