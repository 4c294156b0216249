/*
 * ar.h -- C-ABI of the MI355X (gfx950) multi-buffer all-reduce core.
 *
 * On one GPU, P simulated rank buffers of bf16 activations live in that GPU's
 * HBM.  The library sums them element by element with binary32 accumulation
 * in a fixed schedule order and writes bf16 results.  Every entry point
 * launches hand-written HIP kernels on the caller's stream and returns at
 * once; nothing here synchronises or copies between host and device, and the
 * library makes no memory allocation of its own, host or device (the tuning
 * knob ar_set_launch_shape excepted: it allocates a small host table per GPU
 * in use).
 *
 * Pages cited (titles as printed on the pages):
 *   [TBO-AR] "[DSV4] perf(tbo): overlap pure-TP all_reduce on TBO + Delay TP"
 *   [CAR]    "fix(custom_all_reduce): use SYSTEM scope + ACQUIRE ordering for
 *             cross-device signal loads"
 *   [NVRAR]  "Technical Summary: Understanding and Improving Communication
 *             Performance in Multi-node LLM Inference"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - bf16 data is passed as raw 16-bit patterns; payload words as uint64.
 * - Every data pointer is a DEVICE pointer on the current HIP device and must
 *   be 16-byte aligned (AR_ERR_ALIGN otherwise).  Pointer arrays (ins, outs,
 *   in_words, ...) are HOST arrays of device pointers; the library copies the
 *   pointers into kernel arguments, so the host arrays may be freed on return.
 * - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 * - The caller owns every buffer.  The library keeps no pointer after return.
 * - All argument checks, and the size check of every launch grid, happen
 *   before the first launch: AR_ERR_INVALID, AR_ERR_ALIGN, AR_ERR_ALIAS and
 *   AR_ERR_UNSUPPORTED mean no work was queued.  AR_ERR_HIP reports a
 *   failure of the HIP runtime itself; from an entry point that makes
 *   several launches (the staged two-stage, the staged recursive doubling,
 *   the ubatch reduces) it may leave the launches before the failing one
 *   queued.  n == 0 queues nothing and returns AR_OK.
 * - Aliasing: an output may be exactly the same buffer as an input (in
 *   place); any partial overlap between an output and another buffer, or
 *   between two outputs, is AR_ERR_ALIAS.  Inputs may alias each other.
 * - Numerics of every sum: binary32 round-to-nearest-even additions,
 *   subnormals kept, no fused multiply-add, ranks added in order 0..P-1
 *   starting from rank 0's value; one bf16 rounding (nearest, ties to even)
 *   at the end; any NaN result is written as 0x7FC0.  The pages fix only
 *   that the models run in bf16 ([NVRAR] Methodology 1, "Models"); this
 *   accumulation order and rounding are this library's stated reading.
 * - Thread safety: every entry point may be called concurrently from several
 *   host threads on different streams.  The only global state is one
 *   immutable launch table per device (CU count and launch shapes), built
 *   in static storage once, under a lock, by the first call on that device -- lazy
 *   initialisation raced by two ubatch threads is the hazard [TBO-AR] review
 *   comments describe -- and read without a lock by every later call.
 */
#ifndef AR_H_
#define AR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define AR_OK               0
#define AR_ERR_INVALID     -1  /* NULL pointer, P out of range, bad size/split */
#define AR_ERR_ALIGN       -2  /* a data pointer is not 16-byte aligned        */
#define AR_ERR_ALIAS       -3  /* partial overlap between buffers              */
#define AR_ERR_UNSUPPORTED -4  /* e.g. recursive doubling with P not 2^k       */
#define AR_ERR_HIP         -5  /* a HIP runtime call or kernel launch failed   */
#define AR_ERR_SIZE        -6  /* n beyond the library's static scratch        */

#define AR_MAX_RANKS 8         /* simulated ranks per call: 1..8               */

/* ubatch variants */
#define AR_VARIANT_ONESHOT  0
#define AR_VARIANT_2STAGE   1
#define AR_UBATCH_BOUNDED   256    /* flag, OR-ed into a ubatch variant          */

/* recursive-doubling flags */
#define AR_RD_STAGED        1  /* one launch per exchange step via a mailbox   */
#define AR_RD_FP32_CARRY    2  /* keep binary32 partials between steps (fused) */

/* Human-readable name of a status code (static storage, never NULL). */
const char* ar_status_str(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int ar_version(void);

/*
 * One-shot reduce.  out[i] = rn(((x_0[i] + x_1[i]) + ...) + x_{P-1}[i]).
 * The single-stage counterpart of the two-stage kernel of [CAR] ("Root
 * cause"/"Changes" 3): one rank reads every rank's buffer and sums; one
 * output buffer.
 *   ins    host array of P device pointers, each n bf16 values
 *   P      1..AR_MAX_RANKS (P == 1 copies)
 *   out    device buffer of n bf16; may equal one of ins[] exactly
 *   n      elements per buffer (any n >= 0; no multiple-of-8 requirement)
 * Errors: AR_ERR_INVALID, AR_ERR_ALIGN, AR_ERR_ALIAS, AR_ERR_HIP.
 */
int ar_reduce_oneshot(const void* const* ins, int P, void* out, size_t n, void* stream);

/*
 * Two-stage reduce ([CAR] "Changes" 3, the 2-stage write-mode kernel; [NVRAR]
 * Methodology 3, phases 1 "Reduce-Scatter" and 3 "All-Gather").  All-reduce
 * semantics: every outs[r] receives the same sum as ar_reduce_oneshot.
 *   scratch == NULL  fused: each reduced group of 8 elements is stored
 *                    straight into all P outputs (write mode).
 *   scratch != NULL  staged: launch 1 reduces shard s (elements
 *                    [s*S, min(n,(s+1)*S)), S = ceil(ceil(n/8)/P)*8) into
 *                    scratch; launch 2 copies every shard to all P outputs.
 *                    scratch holds n bf16, disjoint from every other buffer,
 *                    and afterwards holds the reduced values.
 *   outs   host array of P device pointers (n bf16 each); outs[r] may equal
 *          an input exactly; outputs must be pairwise disjoint.  With
 *          outs[r] == ins[r] for every r (in place) and n <= AR_SMALL_ELEMS,
 *          the fused form runs under its own launch shape
 *          (AR_KERNEL_2STAGE_INPLACE_SMALL); the result is the same.
 * Errors: as ar_reduce_oneshot.
 */
int ar_reduce_2stage(const void* const* ins, void* const* outs, int P, size_t n,
                     void* scratch, void* stream);

/*
 * Staged two-stage reduce that allocates nothing and takes no workspace: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same result and
 * kernels as ar_reduce_2stage with a scratch buffer, but the scratch is the
 * library's own static device array of AR_STATIC_SCRATCH_ELEMS bf16 values
 * (32 MiB), one per GPU, held from library load until the process ends.
 *   n      at most AR_STATIC_SCRATCH_ELEMS; a larger n returns AR_ERR_SIZE
 *          and queues nothing.
 * Every call on one GPU uses that GPU's one array: calls whose executions
 * overlap on the same GPU (on different streams, or from different threads)
 * race on it and give undefined results.  Calls in stream order are safe.
 * The array keeps the last call's reduced values; nothing in it needs to
 * start at zero (each call writes every element it later reads).
 * Errors: as ar_reduce_2stage, plus AR_ERR_SIZE; AR_ERR_HIP if the array's
 * device address could not be obtained.
 */
#define AR_STATIC_SCRATCH_ELEMS 16777216
int ar_reduce_2stage_static(const void* const* ins, void* const* outs, int P, size_t n, void* stream);

/*
 * Pack bf16 data into fused 8-byte payload words ([NVRAR] Optimizations,
 * "Fused Payloads"): words[j] = (uint64)seq << 32 | x[2j+1] << 16 | x[2j].
 *   x      n bf16 (n must be even: AR_ERR_INVALID otherwise)
 *   words  n/2 uint64, disjoint from x
 * With the default launch shapes the words are written through past the
 * compute die's L2 (store policy 3), so an ar_unpack_fused_wait running on
 * another stream sees each word as soon as it is stored, while the pack is
 * still running.  With a store policy of 0 or 1 (ar_set_launch_shape) a word
 * may stay in the producer's L2 until that cache evicts it or the kernel
 * ends.
 */
int ar_pack_fused(const void* x, uint64_t* words, size_t n, uint32_t seq, void* stream);

/*
 * Unpack payload words and validate their sequence numbers ([NVRAR]
 * Optimizations, "Sequence-Number Synchronization").  x[2j] and x[2j+1] are
 * always written from words[j].  Each wavefront checks its 64 lanes' words
 * against expected_seq with one ballot and updates the counters once:
 *   d_err[0] += number of words whose high 32 bits != expected_seq
 *   d_err[1]  = min(d_err[1], index j of the first such word)
 *   d_err    device array of 2 uint64, 8-byte aligned; initialise it with
 *            ar_err_init (count 0, first UINT64_MAX).  The library only adds
 *            and takes minima; read it after the stream has finished.
 */
int ar_unpack_fused(const uint64_t* words, void* x, size_t n, uint32_t expected_seq,
                    uint64_t* d_err, void* stream);

/*
 * Unpack with a bounded wait for the producer ([NVRAR] Optimizations,
 * "Fused Payloads" and "Sequence-Number Synchronization": the receiver polls
 * its buffer until each payload carries the expected sequence number; no
 * separate signal).  Meant for a producer that writes `words` concurrently,
 * from another stream of the same device (e.g. ar_pack_fused).  Each word is
 * read with a 64-bit agent-scope atomic load, so a word that shows the
 * expected sequence number also shows its data.  A wavefront re-polls its
 * words (sleeping briefly between polls) until all carry expected_seq or
 * until it has polled max_spins times in total; then it writes the data it
 * holds.  The kernel runs on a persistent grid of a few workgroups per CU and
 * requests no LDS, so the producer can always be scheduled beside it.
 *   d_err    as ar_unpack_fused: words whose sequence number still differs
 *            after the wait are counted, with the first index.
 *   max_spins >= 1.  Every wait is bounded: the call always completes.
 * The producer must be able to run while this kernel waits: HIP maps streams
 * onto a few hardware queues, and a producer queued behind this call on the
 * same queue only starts after the wait has run out (its words then count as
 * mismatches).  Queue the producer first, or on a stream known to be on
 * another queue.
 * Errors: as ar_unpack_fused, plus AR_ERR_INVALID for max_spins == 0.
 */
int ar_unpack_fused_wait(const uint64_t* words, void* x, size_t n, uint32_t expected_seq,
                         uint32_t max_spins, uint64_t* d_err, void* stream);

/*
 * Recursive-doubling combine over P = 2, 4 or 8 payload buffers ([NVRAR]
 * Methodology 3, phase 2 "Inter-node Recursive-Doubling", and Optimizations
 * "Fused Payloads" / "Sequence-Number Synchronization").
 * Step k = 0..L-1 (L = log2 P): rank r combines with partner r XOR 2^k.  The
 * received payload must carry seq0 + k; the combined payload carries
 * seq0 + k + 1 (uint32, wrapping).  Default (round each step): the exchanged
 * partial is the bf16 payload, so each combine is rn(f(own) + f(partner)).
 * All P outputs come out bitwise identical (binary32 addition commutes).
 *   in_words, out_words  host arrays of P device pointers, n/2 words each;
 *                        out_words[r] may equal in_words[q] exactly
 *   n        bf16 elements per rank (even)
 *   flags    0: fused -- one launch computes every step in registers.
 *            AR_RD_STAGED: one launch per step; intermediate payloads go
 *              through `mailbox`: P*(L-1)*Ws words with Ws = n/2 rounded up
 *              to even (each rank's slot stays 16-byte aligned), disjoint
 *              from all other buffers; may be NULL when P == 2.
 *            AR_RD_FP32_CARRY (fused only): binary32 partials between steps,
 *              one rounding at the end (the tree order, reordered relative
 *              to the sequential sum).
 *   d_err    as ar_unpack_fused: d_err[0] counts received words whose
 *            sequence number is wrong; d_err[1] = min over them of
 *            (k*P + q)*(n/2) + j, q the rank whose payload was received.
 * Errors: AR_ERR_UNSUPPORTED for P not in {2,4,8} or FP32_CARRY with STAGED,
 *         AR_ERR_INVALID for odd n or a missing mailbox, plus the common ones.
 */
int ar_rd_schedule(const uint64_t* const* in_words, uint64_t* const* out_words, int P,
                   size_t n, uint32_t seq0, uint64_t* mailbox, int flags, uint64_t* d_err,
                   void* stream);

/*
 * Two-stream chunked ubatch reduce ([TBO-AR] pull request overview: the TP
 * all-reduce of each ubatch runs on its own stream so it overlaps the partner
 * ubatch's compute; [NVRAR] Optimizations, "Chunked Non-blocking
 * Communication").  Each rank buffer is a row-major [rows x hidden] bf16
 * matrix.  Rows are split into n_ubatch ubatches (ubatch_rows == NULL: equal
 * split, remainder to the last; otherwise the counts, which must sum to
 * rows).  Ubatch u is reduced on streams[u] in ascending chunks of
 * chunk_bytes of every rank buffer; a chunk is the unit that workgroups are
 * assigned to, and chunks are dispatched in ascending order.
 *   variant  AR_VARIANT_2STAGE: all P outputs; AR_VARIANT_ONESHOT: outs[0]
 *            only (outs[1..] ignored, may be NULL).  Either may be OR-ed
 *            with AR_UBATCH_BOUNDED: each ubatch then runs on a persistent
 *            grid that holds only part of the device (the
 *            AR_KERNEL_UBATCH_BOUNDED launch shape: by default one 512-lane
 *            workgroup on each of half the CUs), walking the same chunks in
 *            the same order.  It is slower alone but leaves the rest of the
 *            device to compute queued beside it on another stream, which is
 *            the point of the two-ubatch overlap.  Results are identical.
 *   chunk_bytes  > 0, a multiple of 16.
 *   streams  host array of n_ubatch hipStream_t (entries may be NULL);
 *            the caller orders them against other work with events.
 *   n_ubatch 1..16.
 * Results are identical to ar_reduce_oneshot for any split and chunk size.
 */
int ar_reduce_ubatch(const void* const* ins, void* const* outs, int P, size_t rows,
                     size_t hidden, int n_ubatch, const size_t* ubatch_rows,
                     size_t chunk_bytes, int variant, void* const* streams);

/*
 * Launch-shape control (tuning; not a step of the reduction).  Every kernel
 * kind runs on a flat grid of `block`-lane workgroups (64, 128 or 256) with
 * optional non-temporal loads (`nt_loads` 0 or 1), an output store policy
 * `stores` -- 0 plain, 1 non-temporal, 2 written through past the compute
 * die's L2 (SC1), 3 SC1 + non-temporal; UNPACK_WAIT uses only the
 * non-temporal bit, UBATCH_FLAGS always writes through -- and at most
 * `wg_per_cu` workgroups per compute unit (0 = no cap; enforced by
 * requesting unused LDS).  `vec` (1 or 2) sets how much each lane handles:
 *   ONESHOT, 2STAGE, UBATCH, UBATCH_FLAGS, RD, QUANT_FP8 and their _SMALL
 *     kinds, 2STAGE_INPLACE_SMALL: vec 16-byte groups per buffer, each a
 *     contiguous span across the wavefront;
 *   PACK, UNPACK and their _SMALL kinds: 1 -> 8 bytes of bf16 (one 16-byte
 *     payload access) per lane, 2 -> 16 bytes of bf16 (two adjacent payload
 *     accesses);
 *   REDUCE_FP8, REDUCE_FP8_ALL: 1 -> 8 elements (one 16-byte store per
 *     output) per lane, 2 -> 16 elements;
 *   RS, AG, RDSTEP, UNPACK_WAIT: ignored.
 * Defaults are the fastest shapes measured on MI355X.  A new shape applies
 * to launches made after the call, process-wide; the call is thread-safe.
 * Returns AR_ERR_INVALID for an unknown kind or out-of-range field.
 *
 * The one-shot, fused two-stage, fused recursive-doubling, staged
 * recursive-doubling-step, pack and unpack kernels have a second kind each
 * (..._SMALL) whose shape applies when a call's element count n is at most
 * AR_SMALL_ELEMS (4 MiB of bf16 per rank: the decode messages); the fused
 * two-stage has a third for such calls made in place
 * (2STAGE_INPLACE_SMALL).  Such a call moves too little data for the
 * occupancy cap that helps long streams; its time is launch, one memory
 * round trip and the number of workgroup rounds, so its default is uncapped
 * with plain loads, which also keep data that is already on chip there (and,
 * for the staged step, plain stores, which keep each step's mailbox on chip
 * for the next step); the in-place kind, which rewrites the lines it has
 * just read, is fastest with non-temporal loads and stores.  With one group per lane, the one-shot, fused
 * two-stage, pack and unpack small kinds launch kernels with a compact
 * argument segment (28-80 bytes, no hidden arguments), which HIP enqueues
 * faster: the host's launch cost bounds a decode-size call made outside a
 * graph.  The fused two-stage with separate outputs passes its buffers as
 * 32-bit offsets from ins[0] in units of the largest power of two dividing
 * every difference; a call with a buffer out of that reach (at least
 * +-32 GiB) takes the general kernel, with the same result.
 */
#define AR_SMALL_ELEMS 2097152
#define AR_KERNEL_ONESHOT  0   /* ar_reduce_oneshot                         */
#define AR_KERNEL_2STAGE   1   /* ar_reduce_2stage, fused                    */
#define AR_KERNEL_UBATCH   2   /* ar_reduce_ubatch, two-stage variant        */
#define AR_KERNEL_RS       3   /* ar_reduce_2stage, staged: reduce-scatter   */
#define AR_KERNEL_AG       4   /* ar_reduce_2stage, staged: all-gather       */
#define AR_KERNEL_PACK     5   /* ar_pack_fused                              */
#define AR_KERNEL_UNPACK   6   /* ar_unpack_fused                            */
#define AR_KERNEL_RD       7   /* ar_rd_schedule, fused                      */
#define AR_KERNEL_RDSTEP   8   /* ar_rd_schedule, staged (per step)          */
#define AR_KERNEL_UNPACK_WAIT 9 /* ar_unpack_fused_wait; wg_per_cu sets the
                                   persistent grid, no LDS is requested      */
#define AR_KERNEL_UBATCH_FLAGS 10 /* ar_reduce_ubatch_flags (both variants)  */
#define AR_KERNEL_QUANT_FP8 11  /* ar_quantize_fp8                          */
#define AR_KERNEL_REDUCE_FP8 12 /* ar_reduce_fp8, one output               */
#define AR_KERNEL_REDUCE_FP8_ALL 13 /* ar_reduce_fp8, P outputs            */
#define AR_KERNEL_ONESHOT_SMALL 14 /* ar_reduce_oneshot, n <= AR_SMALL_ELEMS   */
#define AR_KERNEL_2STAGE_SMALL 15  /* ar_reduce_2stage fused, n <= AR_SMALL_ELEMS */
#define AR_KERNEL_RD_SMALL 16      /* ar_rd_schedule fused, n <= AR_SMALL_ELEMS */
#define AR_KERNEL_RDSTEP_SMALL 17  /* ar_rd_schedule staged, n <= AR_SMALL_ELEMS */
#define AR_KERNEL_PACK_SMALL 18    /* ar_pack_fused, n <= AR_SMALL_ELEMS        */
#define AR_KERNEL_UNPACK_SMALL 19  /* ar_unpack_fused, n <= AR_SMALL_ELEMS      */
#define AR_KERNEL_UBATCH_BOUNDED 20 /* ar_reduce_ubatch with AR_UBATCH_BOUNDED:
                                      block 256, 512 or 1024 lanes; wg_per_cu
                                      (1..8) is the footprint in eighths of
                                      the device: cus * wg_per_cu / 8
                                      workgroups; no LDS is requested    */
#define AR_KERNEL_2STAGE_INPLACE_SMALL 21 /* ar_reduce_2stage fused with
                                      outs[r] == ins[r] for every r,
                                      n <= AR_SMALL_ELEMS: a read-modify-
                                      write of the same lines, tuned apart
                                      from 2STAGE_SMALL                   */
int ar_set_launch_shape(int kind, int block, int vec, int nt_loads, int stores, int wg_per_cu);
int ar_get_launch_shape(int kind, int* block, int* vec, int* nt_loads, int* stores,
                        int* wg_per_cu);

/*
 * Chunked ubatch reduce with per-chunk completion flags ([NVRAR]
 * Optimizations, "Chunked Non-blocking Communication": the next stage starts
 * on a chunk as soon as it is reduced; [TBO-AR] pull request overview: the
 * all-reduce of a ubatch runs beside the partner's compute).  Same work and
 * arguments as ar_reduce_ubatch, plus:
 *   chunk_done   device uint32[n_flags]: entry g is set to `epoch` once
 *                chunk g has been written to every output.  The outputs of a
 *                flagged call are written through to device-coherent memory
 *                (not left dirty in one XCD's L2), and the flag is stored with
 *                a device-scope store only after every workgroup of the chunk
 *                has had its stores acknowledged, so publishing costs no L2
 *                writeback.  Chunks are numbered across ubatches in order,
 *                ubatch 0's first.  A consumer on any stream of the device
 *                polls chunk_done[g] with device-scope loads until it equals
 *                epoch, then performs a device-scope acquire (fence or
 *                acquire load) before reading chunk g of the outputs.  Poll
 *                with relaxed loads and acquire once: an acquire on every
 *                poll invalidates the XCD's L2 each time.  A waiting consumer
 *                must leave the GPU room for the producer's workgroups (a
 *                grid that fills every wave slot keeps them from starting),
 *                and should be queued after the producer: streams can share
 *                a hardware queue.
 *   chunk_tiles  device uint32[n_flags], zero before the first call; every
 *                call leaves it zero again, so it is reused without
 *                re-initialisation.  Calls that overlap in time must not
 *                share it.
 *   n_flags      entries in each array: at least the total chunk count,
 *                the sum over ubatches of ceil(rows_u * hidden * 2 / chunk_bytes).
 *   epoch        nonzero value published by this call (e.g. a call counter).
 * Errors: as ar_reduce_ubatch, plus AR_ERR_INVALID for epoch == 0, a NULL or
 *         too short array, AR_ERR_ALIGN for arrays not 4-byte aligned,
 *         AR_ERR_ALIAS if the arrays overlap each other or a data buffer, and
 *         AR_ERR_UNSUPPORTED for a variant with AR_UBATCH_BOUNDED.
 */
int ar_reduce_ubatch_flags(const void* const* ins, void* const* outs, int P, size_t rows,
                           size_t hidden, int n_ubatch, const size_t* ubatch_rows,
                           size_t chunk_bytes, int variant, void* const* streams,
                           uint32_t* chunk_done, uint32_t* chunk_tiles, size_t n_flags,
                           uint32_t epoch);

/*
 * fp8-quantised contributions ([TBO-AR] reviewed diff: the custom
 * all-reduce call site passes a ca_fp8_quant flag; the page gives no
 * scheme, so the following is this library's reading).  A rank's bf16
 * buffer travels as E4M3 codes -- the OCP "FN" encoding: bias 7, no
 * infinities, 0x7F / 0xFF are NaN, largest finite 448 -- with one
 * power-of-two scale per block of 32 consecutive elements (the block and
 * scale layout of the OCP Microscaling formats).
 *
 * ar_quantize_fp8: for each of the P buffers xs[p] (n bf16 elements):
 *   scales[p][b] = k_b + 127, where k_b is the smallest integer in
 *                  [-127, 127] with max |x_i| <= 448 * 2^k_b over the finite
 *                  elements of block b (elements 32b .. min(32b+32, n)-1;
 *                  0 if none); so no element is clipped.
 *   codes[p][i]  = the E4M3 code nearest to x_i / 2^k_b (ties to even
 *                  mantissa; the sign is kept, so -0 and negative values that
 *                  round to zero give 0x80); a NaN or infinite x_i gives 0x7F.
 *   xs, codes   host arrays of P device pointers; xs[p] and codes[p] 16-byte
 *               aligned, codes[p] n bytes.
 *   scales      host array of P device pointers, ceil(n/32) bytes each, any
 *               alignment.
 * All P buffers are quantised by one launch.  No code or scale buffer may
 * overlap an input or another code / scale buffer.
 *
 * ar_reduce_fp8: out[i] = rn(((d_0 + d_1) + d_2) + ... + d_{P-1}), where
 *   d_p = value(codes[p][i]) * 2^(scales[p][i/32] - 127) is exact in
 *   binary32 (only an element of magnitude >= 1.9375 * 2^127, the top 8
 *   finite bf16 values, dequantises to infinity: its code is 256 at scale
 *   2^120), the sums are binary32 in rank order and rn is the same bf16
 *   rounding as ar_reduce_oneshot (NaN -> 0x7FC0; a NaN code poisons its
 *   element).  n_out == 1: outs[0] only (one rank's share); n_out == P:
 *   every outs[r] gets the sum (all-reduce write mode).  outs[] 16-byte
 *   aligned, n bf16 each, disjoint from each other and from every code and
 *   scale buffer.
 * Errors (both): AR_ERR_INVALID for NULL pointers, P outside [1, 8] or
 *   n_out not in {1, P}; AR_ERR_ALIGN; AR_ERR_ALIAS.  n == 0 queues nothing.
 */
int ar_quantize_fp8(const void* const* xs, uint8_t* const* codes, uint8_t* const* scales, int P,
                    size_t n, void* stream);
int ar_reduce_fp8(const uint8_t* const* codes, const uint8_t* const* scales, int P, void* const* outs,
                  int n_out, size_t n, void* stream);

/*
 * Initialise an error record for ar_unpack_fused / ar_rd_schedule on
 * `stream`: d_err[0] = 0, d_err[1] = UINT64_MAX.  Uses a one-thread kernel,
 * not a memset, so it may be recorded in a HIP graph.
 */
int ar_err_init(uint64_t* d_err, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* AR_H_ */
