"""GPU parity of every hot-path call against the CPU oracle, through the C-ABI.

Matched order (one-shot, two-stage, ubatch vs the sequential oracle; RD vs
the oracle's RD): bit-exact.  Sequence numbers, mismatch counts and first
indices: exact.  Every size compares every element: the full-size
configurations download their inputs and outputs block by block and run the
oracle on each block over host threads.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_amd as tar
from tensor_all_reduce_amd import synth
from gpu_util import (DEV, note, up16, down16, up64, down64, empty16, new_err, err_host, bits16,
                      blocks, down16_range, down64_range, pmap_slices, first_mismatch)

pytestmark = pytest.mark.gpu

HIDDEN = 8192


def check_full(got: torch.Tensor, want: np.ndarray, what: str):
    g = down16(got)
    bad = np.nonzero(g != want)[0]
    assert bad.size == 0, (f"{what}: {bad.size} mismatches, first at {bad[0]}: "
                           f"got 0x{int(g[bad[0]]):04X} want 0x{int(want[bad[0]]):04X}")


# ------------------------------------------------------------ one-shot / two-stage

@pytest.mark.parametrize("P,n", [(2, HIDDEN)] + [(8, T * HIDDEN) for T in (8, 32, 128)])
def test_decode_configs(P, n):
    """P=2 [1 x 8192] and P=8 [T x 8192], T in {8, 32, 128}: one-shot,
    two-stage fused and staged, N(0,1) inputs."""
    cfg, tag = (1, 0) if P == 2 else (2, n // HIDDEN)
    xs = synth.rank_buffers("normal", P, n, cfg, tag)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    note(f"oneshot P={P} n={n}")
    out = empty16(n)
    tar.ar_reduce_oneshot(ins, out)
    torch.cuda.synchronize()
    check_full(out, ref, "oneshot")
    note(f"2stage fused P={P} n={n}")
    outs = [empty16(n) for _ in range(P)]
    tar.ar_reduce_2stage(ins, outs)
    torch.cuda.synchronize()
    for o in outs:
        check_full(o, ref, "2stage fused")
    note(f"2stage staged P={P} n={n}")
    outs2 = [empty16(n) for _ in range(P)]
    scratch = empty16(n)
    tar.ar_reduce_2stage(ins, outs2, scratch=scratch)
    torch.cuda.synchronize()
    check_full(scratch, ref, "staged scratch")
    for o in outs2:
        check_full(o, ref, "2stage staged")


# the last three sit on and around the element count at which the one-shot and
# two-stage calls switch from their small-message launch shape to the large one
RAGGED = [1, 2, 7, 8, 9, 15, 17, 255, 1000, 2049, 65536 + 3, 300001, 4 * 1024 * 1024 + 5,
          tar.AR_SMALL_ELEMS - 1, tar.AR_SMALL_ELEMS, tar.AR_SMALL_ELEMS + 1]


@pytest.mark.parametrize("n", RAGGED)
@pytest.mark.parametrize("P", [1, 2, 3, 5, 8])
def test_ragged_sizes(P, n):
    """Sizes that are not multiples of the 8-element group, spanning one
    partial group up to several grid-stride passes."""
    xs = synth.rank_buffers("logmag", P, n, 20, n)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    note(f"ragged P={P} n={n}")
    out = empty16(n)
    tar.ar_reduce_oneshot(ins, out)
    outs = [empty16(n) for _ in range(P)]
    tar.ar_reduce_2stage(ins, outs)
    outs2 = [empty16(n) for _ in range(P)]
    tar.ar_reduce_2stage(ins, outs2, scratch=empty16(n))
    torch.cuda.synchronize()
    check_full(out, ref, "oneshot")
    for o in outs + outs2:
        check_full(o, ref, "2stage")


SPECIALS = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80,
                     0x7FC0, 0x7F81, 0xFFC1, 0x3F80, 0xBF80, 0x4B80, 0xCB80, 0x3B80, 0x3380],
                    dtype=np.uint16)


@pytest.mark.parametrize("P", [2, 3, 8])
def test_special_values(P):
    """NaN payloads, infinities, signed zeros, subnormals, values at the
    overflow edge and absorption cases, densely mixed into the inputs."""
    n = 200003
    xs = synth.rank_buffers("logmag", P, n, 21, P)
    g = np.random.default_rng([22, P])
    for x in xs:
        idx = g.choice(n, size=n // 3, replace=False)
        x[idx] = g.choice(SPECIALS, size=idx.size)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    note(f"special values P={P}")
    out = empty16(n)
    tar.ar_reduce_oneshot(ins, out)
    outs = [empty16(n) for _ in range(P)]
    tar.ar_reduce_2stage(ins, outs, scratch=empty16(n))
    torch.cuda.synchronize()
    check_full(out, ref, "oneshot specials")
    for o in outs:
        check_full(o, ref, "2stage specials")


def test_exhaustive_pairs_p2():
    """P=2: every bf16 pattern against 19 special and 45 random partners."""
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    partners = np.concatenate([SPECIALS, synth.normal(45, 23)])
    A = np.tile(a, partners.size)
    Bv = np.repeat(partners, a.size)
    ref = oracle.reduce_seq([A, Bv])
    note("exhaustive pairs P=2")
    out = empty16(A.size)
    tar.ar_reduce_oneshot([up16(A), up16(Bv)], out)
    torch.cuda.synchronize()
    check_full(out, ref, "pairs")


def test_in_place():
    P, n = 8, 123457
    xs = synth.rank_buffers("normal", P, n, 24)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    note("in-place 2stage fused")
    tar.ar_reduce_2stage(ins, ins)
    torch.cuda.synchronize()
    for t in ins:
        check_full(t, ref, "in-place fused")
    ins = [up16(x) for x in xs]
    note("in-place 2stage staged")
    tar.ar_reduce_2stage(ins, ins, scratch=empty16(n))
    torch.cuda.synchronize()
    for t in ins:
        check_full(t, ref, "in-place staged")
    ins = [up16(x) for x in xs]
    note("in-place oneshot")
    tar.ar_reduce_oneshot(ins, ins[3])
    torch.cuda.synchronize()
    check_full(ins[3], ref, "in-place oneshot")


@pytest.mark.parametrize("n", [3 * 8192 + 5, tar.AR_SMALL_ELEMS + 1001])
def test_mixed_aliasing(n):
    """Outputs that are partly the inputs themselves: ranks 0, 2, 4, 6 write
    into their own input, rank 1 into rank 5's input, ranks 3, 5, 7 into
    separate buffers (pairwise disjoint outputs, each equal to an input or
    apart from all).  Fused (the compact offset kernel below
    AR_SMALL_ELEMS, k_reduce above), staged and static-scratch two-stage;
    every output matches the oracle."""
    P = 8
    xs = synth.rank_buffers("normal", P, n, 6, n)
    ref = oracle.reduce_seq(xs)
    for mode in ("fused", "staged", "static"):
        if mode == "static" and n > tar.AR_STATIC_SCRATCH_ELEMS:
            continue
        ins = [up16(x) for x in xs]
        sep = {r: empty16(n) for r in (3, 5, 7)}
        outs = [ins[0], ins[5], ins[2], sep[3], ins[4], sep[5], ins[6], sep[7]]
        note(f"mixed aliasing n={n} {mode}")
        if mode == "fused":
            tar.ar_reduce_2stage(ins, outs)
        elif mode == "staged":
            tar.ar_reduce_2stage(ins, outs, scratch=empty16(n))
        else:
            tar.ar_reduce_2stage_static(ins, outs)
        torch.cuda.synchronize()
        for r, o in enumerate(outs):
            check_full(o, ref, f"mixed aliasing n={n} {mode}: rank {r}")


def test_small_2stage_buffer_offsets():
    """The small fused two-stage with separate outputs passes its buffers to
    the kernel as signed 32-bit offsets from ins[0], in units of the largest
    power of two dividing every difference, and takes the general kernel when
    one does not fit.  All buffers are carved from one 33 GiB allocation, with
    outs[0] moved: 128 KiB before ins[0] (a negative offset, 128 KiB units),
    3 GiB plus 16 bytes past it (16-byte units, the smallest the alignment rule
    allows; still within reach) and 33 GiB plus 16 bytes past it (beyond the
    +-32 GiB reach of 16-byte units: the general kernel).  Each matches the
    oracle."""
    P, n = 8, 3 * 8192 + 5
    S = 1 << 16                                    # element stride between carved buffers (128 KiB)
    xs = synth.rank_buffers("normal", P, n, 4, 777)
    ref = oracle.reduce_seq(xs)
    near, far = (3 << 30) // 2 + 8, (33 << 30) // 2 + 8   # in elements
    big = torch.empty(far + n, dtype=torch.int16, device=DEV)
    try:
        ins = [big[(1 + p) * S:(1 + p) * S + n] for p in range(P)]
        for t, x in zip(ins, xs):
            t.copy_(up16(x))
        for out0_at, what in ((0, "outs[0] 128 KiB before ins[0]"), (near, "outs[0] 3 GiB + 16 B past ins[0]"),
                              (far, "outs[0] 33 GiB + 16 B past ins[0]")):
            outs = [big[out0_at:out0_at + n]] + [big[(1 + P + p) * S:(1 + P + p) * S + n] for p in range(1, P)]
            for o in outs:
                o.fill_(0x5A5A)
            note(f"small two-stage, buffer offsets: {what}")
            tar.ar_reduce_2stage(ins, outs)
            torch.cuda.synchronize()
            for r, o in enumerate(outs):
                check_full(o, ref, f"{what}: rank {r}")
    finally:
        del big
        torch.cuda.empty_cache()


def test_prepared_calls():
    """Every hot-path call prepared once (tar.prepare) and then called on two
    input sets written into the same tensors, one handle on a side stream:
    each result matches the oracle, so a handle reuses its pointers and reads
    the buffers' current contents."""
    P, n = 8, 4 * 8192 + 13
    n2 = n - 1                                   # payload path: an even element count
    ins = [empty16(n) for _ in range(P)]
    bufs = [empty16(n) for _ in range(P)]
    out1, outs, outs2, scr = empty16(n), [empty16(n) for _ in range(P)], [empty16(n) for _ in range(P)], empty16(n)
    words = [torch.empty(n2 // 2, dtype=torch.int64, device=DEV) for _ in range(P)]
    rdo = [torch.empty_like(w) for w in words]
    x3, err = empty16(n2), torch.empty(2, dtype=torch.int64, device=DEV)
    codes = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(P)]
    scales = [torch.empty(tar.fp8_scale_count(n), dtype=torch.uint8, device=DEV) for _ in range(P)]
    side = torch.cuda.Stream()
    h = {"oneshot": tar.prepare(tar.ar_reduce_oneshot, ins, out1),
         "fused": tar.prepare(tar.ar_reduce_2stage, ins, outs, stream=side),
         "staged": tar.prepare(tar.ar_reduce_2stage, ins, outs2, scratch=scr),
         "inplace": tar.prepare(tar.ar_reduce_2stage, bufs, bufs),
         "err": tar.prepare(tar.ar_err_init, err),
         "pack": [tar.prepare(tar.ar_pack_fused, ins[r], words[r], 9, n=n2) for r in range(P)],
         "rd": tar.prepare(tar.ar_rd_schedule, words, rdo, 9, err),
         "unpack": tar.prepare(tar.ar_unpack_fused, rdo[6], x3, 12, err, n=n2),
         "quant": tar.prepare(tar.ar_quantize_fp8, ins, codes, scales),
         "fp8": tar.prepare(tar.ar_reduce_fp8, codes, scales, [out1])}
    for tag in (0, 1):
        xs = synth.rank_buffers("normal", P, n, 31, tag)
        ref = oracle.reduce_seq(xs)
        for t, b, x in zip(ins, bufs, xs):
            t.copy_(up16(x))
            b.copy_(up16(x))
        torch.cuda.synchronize()
        note(f"prepared calls, input set {tag}")
        h["oneshot"]()
        h["staged"]()
        h["inplace"]()
        side.wait_stream(torch.cuda.current_stream())
        h["fused"]()
        torch.cuda.current_stream().wait_stream(side)
        h["err"]()
        for hp in h["pack"]:
            hp()
        h["rd"]()
        h["unpack"]()
        torch.cuda.synchronize()
        check_full(out1, ref, f"prepared oneshot, set {tag}")
        for r in range(P):
            check_full(outs[r], ref, f"prepared fused, set {tag}, rank {r}")
            check_full(outs2[r], ref, f"prepared staged, set {tag}, rank {r}")
            check_full(bufs[r], ref, f"prepared in place, set {tag}, rank {r}")
        o_words, _ = oracle.rd([oracle.pack(v[:n2], 9) for v in xs], 9)
        want, _ = oracle.unpack(o_words[6], 12)
        check_full(x3, want, f"prepared pack/RD/unpack, set {tag}")
        assert err_host(err)[0] == 0
        h["quant"]()
        h["fp8"]()
        torch.cuda.synchronize()
        q = [oracle.quant_fp8(v) for v in xs]
        check_full(out1, oracle.reduce_fp8([c for c, _ in q], [s_ for _, s_ in q]), f"prepared fp8, set {tag}")


def test_canaries_untouched():
    """Outputs carved out of larger buffers: the guard bytes around them keep
    their pattern, so no kernel writes outside [0, n)."""
    P, n, G = 8, 50001, 4096
    xs = synth.rank_buffers("normal", P, n, 25)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    pattern = np.int16(0x5A5A)
    bigs = [torch.full((n + 2 * G,), int(pattern), dtype=torch.int16, device=DEV) for _ in range(P)]
    outs = [b[G:G + n] for b in bigs]
    sbig = torch.full((n + 2 * G,), int(pattern), dtype=torch.int16, device=DEV)
    note("canaries")
    tar.ar_reduce_2stage(ins, outs, scratch=sbig[G:G + n])
    tar.ar_reduce_oneshot(ins, outs[0])
    torch.cuda.synchronize()
    for b in bigs + [sbig]:
        h = down16(b)
        assert np.all(h[:G] == np.uint16(0x5A5A)) and np.all(h[G + n:] == np.uint16(0x5A5A))
        check_full(b[G:G + n], ref, "canary body")


@pytest.mark.parametrize("P,n", [(8, 10), (8, 13), (3, 17), (8, 8 * 8 + 5), (7, 1000 * 7 + 3)])
def test_staged_ragged_tail_canaries(P, n):
    """The staged two-stage where n is not a multiple of 8 and trailing
    shards are empty (n = 10 with P = 8 leaves shards 1..7 empty): only the
    last non-empty shard writes the ragged tail.  Outputs and scratch are
    carved out of guarded buffers; the guards keep their pattern, and every
    output, the scratch, and the static-scratch entry point equal the oracle."""
    G = 256
    xs = synth.rank_buffers("normal", P, n, 26, n)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    bigs = [torch.full((n + 2 * G,), 0x5A5A, dtype=torch.int16, device=DEV) for _ in range(2 * P)]
    outs = [b[G:G + n] for b in bigs[:P]]
    outs2 = [b[G:G + n] for b in bigs[P:]]
    sbig = torch.full((n + 2 * G,), 0x5A5A, dtype=torch.int16, device=DEV)
    note(f"staged ragged tail P={P} n={n}")
    tar.ar_reduce_2stage(ins, outs, scratch=sbig[G:G + n])
    tar.ar_reduce_2stage_static(ins, outs2)
    torch.cuda.synchronize()
    for b in bigs + [sbig]:
        h = down16(b)
        assert np.all(h[:G] == np.uint16(0x5A5A)) and np.all(h[G + n:] == np.uint16(0x5A5A))
        check_full(b[G:G + n], ref, "staged ragged body")


def test_n_zero_is_noop():
    t = empty16(16)
    t.fill_(7)
    note("n=0")
    tar.ar_reduce_oneshot([t, t], t, n=0)
    torch.cuda.synchronize()
    assert np.all(down16(t) == 7)


# ------------------------------------------------------------ pack / RD / unpack

def _rd_case(P, n, seq0, kind="normal", cfg=3):
    xs = synth.rank_buffers(kind, P, n, cfg, P, seq0 & 0xFF)
    return xs, [oracle.pack(x, seq0) for x in xs]


@pytest.mark.parametrize("seq0", [1, 0xFFFFFFFE])
@pytest.mark.parametrize("P,n", [(8, 128 * HIDDEN), (2, 20002), (4, 65538), (8, 6),
                                 (8, tar.AR_SMALL_ELEMS), (8, tar.AR_SMALL_ELEMS + 2)])
def test_pack_rd_unpack(P, n, seq0):
    """Pack on the GPU, recursive doubling (fused R1, staged R1, fused R2),
    unpack with validation; payload words, data and counts vs the oracle."""
    xs, owords = _rd_case(P, n, seq0)
    L = {2: 1, 4: 2, 8: 3}[P]
    ins = [up16(x) for x in xs]
    words = [torch.empty(n // 2, dtype=torch.int64, device=DEV) for _ in range(P)]
    note(f"pack P={P} n={n} seq0={seq0:#x}")
    for i in range(P):
        tar.ar_pack_fused(ins[i], words[i], seq0)
    torch.cuda.synchronize()
    for i in range(P):
        assert np.array_equal(down64(words[i]), owords[i])
    for flags, carry in ((0, False), (tar.AR_RD_STAGED, False), (tar.AR_RD_FP32_CARRY, True)):
        ref_w, ref_e = oracle.rd(owords, seq0, carry)
        out = [torch.empty(n // 2, dtype=torch.int64, device=DEV) for _ in range(P)]
        mb = None
        if flags & tar.AR_RD_STAGED and P > 2:
            mb = torch.empty(tar.rd_mailbox_words(P, n), dtype=torch.int64, device=DEV)
        err = new_err()
        note(f"rd P={P} n={n} flags={flags}")
        tar.ar_rd_schedule(words, out, seq0, err, mailbox=mb, flags=flags)
        torch.cuda.synchronize()
        assert err_host(err) == (int(ref_e[0]), int(ref_e[1])) == (0, 2 ** 64 - 1)
        for r in range(P):
            got = down64(out[r])
            bad = np.nonzero(got != ref_w[r])[0]
            assert bad.size == 0, f"flags={flags} rank {r}: word {bad[0]} {got[bad[0]]:#x} vs {ref_w[r][bad[0]]:#x}"
        x = empty16(n)
        err2 = new_err()
        note(f"unpack P={P} n={n}")
        tar.ar_unpack_fused(out[P - 1], x, (seq0 + L) & 0xFFFFFFFF, err2)
        torch.cuda.synchronize()
        ox, oe = oracle.unpack(ref_w[P - 1], (seq0 + L) & 0xFFFFFFFF)
        check_full(x, ox, "unpack")
        assert err_host(err2) == (int(oe[0]), int(oe[1]))


@pytest.mark.parametrize("P,n", [(2, 24590), (4, 24590), (8, 24590), (8, 128 * HIDDEN)])
def test_rd_outputs_alias_inputs(P, n):
    """Recursive doubling with out_words equal to in_words: in place, and
    permuted (rank r's result in rank P-1-r's input).  Fused R1, staged R1
    (P = 2 in one launch, no mailbox) and fused R2; every output word and
    the error record match the oracle.  n/2 is odd for the small sizes, so
    the tail word is handled too."""
    seq0 = 77
    xs, owords = _rd_case(P, n, seq0, cfg=34)
    for flags, carry in ((0, False), (tar.AR_RD_STAGED, False), (tar.AR_RD_FP32_CARRY, True)):
        ref_w, ref_e = oracle.rd(owords, seq0, carry)
        for layout in ("in place", "permuted"):
            words = [up64(w) for w in owords]
            out = words if layout == "in place" else words[::-1]
            mb = None
            if flags & tar.AR_RD_STAGED and P > 2:
                mb = torch.empty(tar.rd_mailbox_words(P, n), dtype=torch.int64, device=DEV)
            err = new_err()
            note(f"rd aliasing P={P} n={n} flags={flags} {layout}")
            tar.ar_rd_schedule(words, out, seq0, err, mailbox=mb, flags=flags)
            torch.cuda.synchronize()
            assert err_host(err) == (int(ref_e[0]), int(ref_e[1])) == (0, 2 ** 64 - 1)
            for r in range(P):
                got = down64(out[r])
                bad = np.nonzero(got != ref_w[r])[0]
                assert bad.size == 0, (f"{layout} flags={flags} rank {r}: word {bad[0]} "
                                       f"{got[bad[0]]:#x} vs {ref_w[r][bad[0]]:#x}")


@pytest.mark.parametrize("staged", [False, True])
def test_rd_error_counts(staged):
    """Host-forced faults: corrupted sequence numbers in chosen words of
    chosen ranks are counted exactly and the first index is exact; the data
    is still combined from the payload bits, as in the oracle."""
    P, n, seq0 = 8, 128 * HIDDEN, 40
    xs, owords = _rd_case(P, n, seq0, cfg=31)
    W = n // 2
    hits = [(5, 7), (5, W - 1), (2, 1000), (7, 0), (0, W // 2)]
    for r, j in hits:
        owords[r][j] = (owords[r][j] & np.uint64(0xFFFFFFFF)) | (np.uint64(seq0 + 9) << np.uint64(32))
    ref_w, ref_e = oracle.rd(owords, seq0)
    words = [up64(w) for w in owords]
    out = [torch.empty(W, dtype=torch.int64, device=DEV) for _ in range(P)]
    mb = torch.empty(tar.rd_mailbox_words(P, n), dtype=torch.int64, device=DEV) if staged else None
    err = new_err()
    note(f"rd faults staged={staged}")
    tar.ar_rd_schedule(words, out, seq0, err, mailbox=mb, flags=tar.AR_RD_STAGED if staged else 0)
    torch.cuda.synchronize()
    assert err_host(err) == (len(hits), min(r * W + j for r, j in hits))
    assert (int(ref_e[0]), int(ref_e[1])) == err_host(err)
    for r in range(P):
        assert np.array_equal(down64(out[r]), ref_w[r])


def test_unpack_faults():
    """Stale payload (previous sequence number), a wrong expected number,
    and k corrupted words: exact counts and first indices."""
    n = 2 * HIDDEN * 64 + 6
    x = synth.normal(n, 32)
    w = oracle.pack(x, 100)
    g = np.random.default_rng(33)
    bad = np.sort(g.choice(w.size, size=77, replace=False))
    wc = w.copy()
    wc[bad] ^= np.uint64(1) << np.uint64(40)
    for words, expect, count, first in ((w, 100, 0, 2 ** 64 - 1), (oracle.pack(x, 99), 100, w.size, 0),
                                        (w, 101, w.size, 0), (wc, 100, 77, int(bad[0]))):
        out = empty16(n)
        err = new_err()
        note(f"unpack fault expect={expect} count={count}")
        tar.ar_unpack_fused(up64(words), out, expect, err)
        torch.cuda.synchronize()
        assert err_host(err) == (count, first)
        check_full(out, x, "unpack data")
    # counters accumulate across calls and keep the minimum index
    err = new_err()
    out = empty16(n)
    tar.ar_unpack_fused(up64(wc), out, 100, err)
    tar.ar_unpack_fused(up64(oracle.pack(x, 99)), out, 100, err)
    torch.cuda.synchronize()
    assert err_host(err) == (77 + w.size, 0)


# ------------------------------------------------------------ ubatch

@pytest.mark.parametrize("chunk_bytes", [1 << 20, 65536, 4096 + 16, 16])
@pytest.mark.parametrize("split", [None, [3, 61], [64, 0]])
def test_ubatch_small(chunk_bytes, split):
    P, rows, hidden = 8, 64, 1000
    n = rows * hidden
    xs = synth.rank_buffers("logmag", P, n, 5, rows)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    outs = [empty16(n) for _ in range(P)]
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in s:
        st.wait_stream(torch.cuda.current_stream())
    note(f"ubatch rows={rows} hidden={hidden} chunk={chunk_bytes} split={split}")
    tar.ar_reduce_ubatch(ins, outs, rows, hidden, 2, split, chunk_bytes, tar.AR_VARIANT_2STAGE, s)
    one = [empty16(n)] + [None] * (P - 1)
    tar.ar_reduce_ubatch(ins, one, rows, hidden, 2, split, chunk_bytes, tar.AR_VARIANT_ONESHOT, s)
    torch.cuda.synchronize()
    for o in outs:
        check_full(o, ref, "ubatch 2stage")
    check_full(one[0], ref, "ubatch oneshot")


def test_ubatch_many_ubatches_hidden_not_multiple_of_8():
    P, rows, hidden = 5, 37, 1001
    n = rows * hidden
    xs = synth.rank_buffers("normal", P, n, 6)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    outs = [empty16(n) for _ in range(P)]
    streams = [torch.cuda.Stream() for _ in range(3)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    note("ubatch 3 ubatches hidden=1001")
    tar.ar_reduce_ubatch(ins, outs, rows, hidden, 3, None, 4096, tar.AR_VARIANT_2STAGE, streams)
    torch.cuda.synchronize()
    for o in outs:
        check_full(o, ref, "ubatch odd hidden")


@pytest.mark.parametrize("shape", [(512, 1, 1, 1, 4), (256, 2, 1, 3, 1), (1024, 1, 0, 0, 8), (512, 2, 1, 2, 3)])
@pytest.mark.parametrize("chunk_bytes", [1 << 20, 4096 + 16])
def test_ubatch_bounded(shape, chunk_bytes):
    """The bounded-footprint ubatch reduce (AR_UBATCH_BOUNDED): a persistent
    grid of a fraction of the CUs walks the chunked tiles.  Several grid
    shapes (256..1024 lanes, 1/8..8/8 of the CUs, both lane widths, every
    store policy), ragged chunks, three ubatches, hidden not a multiple of 8,
    both variants: bit-exact against the oracle."""
    P, rows, hidden = 8, 512, 8192 + 5
    n = rows * hidden
    xs = synth.rank_buffers("logmag", P, n, 5, 2, shape[0], shape[4])
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    outs = [empty16(n) for _ in range(P)]
    one = [empty16(n)]
    streams = [torch.cuda.Stream() for _ in range(3)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    default = tar.ar_get_launch_shape(tar.AR_KERNEL_UBATCH_BOUNDED)
    tar.ar_set_launch_shape(tar.AR_KERNEL_UBATCH_BOUNDED, *shape)
    try:
        note(f"ubatch bounded shape={shape} chunk={chunk_bytes}")
        tar.ar_reduce_ubatch(ins, outs, rows, hidden, 3, [100, 300, 112], chunk_bytes,
                             tar.AR_VARIANT_2STAGE | tar.AR_UBATCH_BOUNDED, streams)
        tar.ar_reduce_ubatch(ins, one, rows, hidden, 3, [100, 300, 112], chunk_bytes,
                             tar.AR_VARIANT_ONESHOT | tar.AR_UBATCH_BOUNDED, streams)
        torch.cuda.synchronize()
    finally:
        tar.ar_set_launch_shape(tar.AR_KERNEL_UBATCH_BOUNDED, *default)
    for o in outs:
        check_full(o, ref, f"ubatch bounded {shape} 2stage")
    check_full(one[0], ref, f"ubatch bounded {shape} oneshot")


@pytest.mark.parametrize("mode", ["flat", "bounded", "flags", "oneshot", "mixed"])
def test_ubatch_outputs_alias_inputs(mode):
    """The ubatch reduce with outputs that are the inputs: every output its
    own input on the flat grid, the bounded grid and with completion flags;
    the one-shot variant writing into one rank's input; and outputs that are
    partly the inputs (own and another rank's) beside separate buffers."""
    P, rows, hidden = 4, 96, 4096
    n = rows * hidden
    xs = synth.rank_buffers("normal", P, n, 5, 3)
    ref = oracle.reduce_seq(xs)
    bufs = [up16(x) for x in xs]
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in s:
        st.wait_stream(torch.cuda.current_stream())
    note(f"ubatch outputs alias inputs: {mode}")
    if mode == "flat":
        outs = bufs
        tar.ar_reduce_ubatch(bufs, outs, rows, hidden, 2, None, 1 << 16, tar.AR_VARIANT_2STAGE, s)
    elif mode == "bounded":
        outs = bufs
        tar.ar_reduce_ubatch(bufs, outs, rows, hidden, 2, None, 1 << 16,
                             tar.AR_VARIANT_2STAGE | tar.AR_UBATCH_BOUNDED, s)
    elif mode == "flags":
        outs = bufs
        nf = tar.ubatch_chunk_count(rows, hidden, 2, None, 1 << 16)
        done = torch.zeros(nf, dtype=torch.int32, device=DEV)
        tiles = torch.zeros(nf, dtype=torch.int32, device=DEV)
        torch.cuda.synchronize()
        tar.ar_reduce_ubatch_flags(bufs, outs, rows, hidden, done, tiles, 3, 2, None, 1 << 16,
                                   tar.AR_VARIANT_2STAGE, s)
    elif mode == "oneshot":
        outs = [bufs[2]]
        tar.ar_reduce_ubatch(bufs, outs, rows, hidden, 2, None, 1 << 16, tar.AR_VARIANT_ONESHOT, s)
    else:
        outs = [bufs[0], bufs[3], empty16(n), empty16(n)]
        tar.ar_reduce_ubatch(bufs, outs, rows, hidden, 2, [37, 59], 4096 + 16, tar.AR_VARIANT_2STAGE, s)
    torch.cuda.synchronize()
    for r, o in enumerate(outs):
        check_full(o, ref, f"ubatch {mode}: output {r}")
    if mode == "flags":
        assert np.all(done.cpu().numpy() == 3) and not tiles.cpu().numpy().any()


# ------------------------------------------------------------ concurrency

def test_two_threads_two_streams():
    """Two host threads, each with its own stream, call concurrently (the
    first calls race the library's one-time device initialisation)."""
    import threading
    P, n = 8, 333333
    xs = synth.rank_buffers("normal", P, n, 7)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    results = {}
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [empty16(n) for _ in range(P)]
                for _ in range(20):
                    tar.ar_reduce_2stage(ins, outs, stream=s)
                    tar.ar_reduce_oneshot(ins, outs[0], stream=s)
                s.synchronize()
                results[k] = [down16(o) for o in outs]
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    torch.cuda.synchronize()
    note("two threads")
    th = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    for k in range(2):
        for o in results[k]:
            assert np.array_equal(o, ref)


# ------------------------------------------------------------ full-size configurations
#
# Every element of every output is compared with the oracle.  The inputs are
# drawn on the GPU (several GiB), downloaded block by block, and the oracle
# runs on each block split over host threads; each output's block is then
# downloaded and compared element for element.

FULL_BLOCK = 1 << 24          # elements per downloaded block (32 MiB per buffer)


def _seq_block(xs):
    return np.concatenate(pmap_slices(oracle.reduce_seq, xs, xs[0].size))


def _compare_full(ins, outputs, n, what):
    """outputs: {name: device tensor of n bf16}; every element of each vs
    oracle.reduce_seq over the same elements of ins.  Returns the number of
    elements compared per output."""
    bad = {}
    for a, b in blocks(n, FULL_BLOCK):
        want = _seq_block([down16_range(x, a, b) for x in ins])
        for name, t in outputs.items():
            cnt, first = first_mismatch(down16_range(t, a, b), want)
            if cnt and name not in bad:
                bad[name] = (a + first, cnt)
            elif cnt:
                bad[name] = (bad[name][0], bad[name][1] + cnt)
    assert not bad, f"{what}: mismatches (first index, count so far) {bad}"
    return n


def test_prefill_2stage_full_size(record_property):
    """P=8 [16384 x 8192] per rank (256 MiB per buffer), N(0,1): every
    element of all P outputs of the fused and the staged two-stage, the
    staged scratch and the one-shot output against the oracle."""
    P, n = 8, 16384 * HIDDEN
    note("prefill full size: generate")
    ins = [bits16(t) for t in synth.device_rank_buffers("normal", P, n, 4)]
    outs = [empty16(n) for _ in range(P)]
    note("prefill full size: 2stage fused")
    tar.ar_reduce_2stage(ins, outs)
    scratch = empty16(n)
    outs2 = [empty16(n) for _ in range(P)]
    note("prefill full size: 2stage staged")
    tar.ar_reduce_2stage(ins, outs2, scratch=scratch)
    one = empty16(n)
    note("prefill full size: oneshot")
    tar.ar_reduce_oneshot(ins, one)
    torch.cuda.synchronize()
    outputs = {f"fused[{r}]": outs[r] for r in range(P)}
    outputs.update({f"staged[{r}]": outs2[r] for r in range(P)})
    outputs.update({"scratch": scratch, "oneshot": one})
    note("prefill full size: compare every element with the oracle")
    _compare_full(ins, outputs, n, "prefill")
    record_property("elements_compared", n * len(outputs))
    print(f"[gpu] prefill full size: {len(outputs)} outputs x {n} elements equal the oracle")
    del ins, outs, outs2, scratch, one
    torch.cuda.empty_cache()


def test_ubatch_full_size(record_property):
    """P=8 [16384 x 16384] per rank split into two 8192-row ubatches on two
    streams, 1 MiB chunks, log-uniform magnitudes in [2^-8, 2^8] with random
    signs: every element of all P outputs of the two-stage variant (flat and
    bounded-footprint grids) and of the one-shot variant's output against
    the oracle."""
    P, rows, hidden = 8, 16384, 16384
    n = rows * hidden
    note("ubatch full size: generate")
    ins = [bits16(t) for t in synth.device_rank_buffers("logmag", P, n, 5)]
    outs = [empty16(n) for _ in range(P)]
    one = empty16(n)
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in s:
        st.wait_stream(torch.cuda.current_stream())
    note("ubatch full size: two-stage variant")
    tar.ar_reduce_ubatch(ins, outs, rows, hidden, 2, None, 1 << 20, tar.AR_VARIANT_2STAGE, s)
    note("ubatch full size: one-shot variant")
    tar.ar_reduce_ubatch(ins, [one], rows, hidden, 2, None, 1 << 20, tar.AR_VARIANT_ONESHOT, s)
    bouts = [empty16(n) for _ in range(P)]
    note("ubatch full size: two-stage variant, bounded footprint")
    tar.ar_reduce_ubatch(ins, bouts, rows, hidden, 2, None, 1 << 20, tar.AR_VARIANT_2STAGE | tar.AR_UBATCH_BOUNDED, s)
    torch.cuda.synchronize()
    outputs = {f"2stage[{r}]": outs[r] for r in range(P)}
    outputs["oneshot"] = one
    outputs.update({f"2stage bounded[{r}]": bouts[r] for r in range(P)})
    note("ubatch full size: compare every element with the oracle")
    _compare_full(ins, outputs, n, "ubatch")
    record_property("elements_compared", n * len(outputs))
    print(f"[gpu] ubatch full size: {len(outputs)} outputs x {n} elements equal the oracle")
    del ins, outs, one, bouts
    torch.cuda.empty_cache()


def test_payload_path_full_size(record_property):
    """The bench's fused-payload rows at their size: P=8 [16384 x 8192] per
    rank (512 MiB of payload per rank), seq0 = 1.  Pack every rank, fused and
    staged recursive doubling, unpack every rank.  Every payload word of
    every rank's pack, fused-RD and staged-RD output, and every element of
    every rank's unpacked output, against the oracle's pack, RD and unpack;
    no sequence mismatch."""
    P, n = 8, 16384 * 8192
    W = n // 2
    note("payload full size: generate")
    ins = [bits16(t) for t in synth.device_rank_buffers("normal", P, n, 9)]
    words = [torch.empty(W, dtype=torch.int64, device=DEV) for _ in range(P)]
    note("payload full size: pack")
    for r in range(P):
        tar.ar_pack_fused(ins[r], words[r], 1)
    rdo = [torch.empty(W, dtype=torch.int64, device=DEV) for _ in range(P)]
    err = new_err()
    note("payload full size: rd fused")
    tar.ar_rd_schedule(words, rdo, 1, err)
    mbox = torch.empty(tar.rd_mailbox_words(P, n), dtype=torch.int64, device=DEV)
    rds = [torch.empty(W, dtype=torch.int64, device=DEV) for _ in range(P)]
    err2 = new_err()
    note("payload full size: rd staged")
    tar.ar_rd_schedule(words, rds, 1, err2, mailbox=mbox, flags=tar.AR_RD_STAGED)
    del mbox
    xo = [empty16(n) for _ in range(P)]
    note("payload full size: unpack")
    for r in range(P):
        tar.ar_unpack_fused(rdo[r], xo[r], 4, err)
    torch.cuda.synchronize()
    assert err_host(err) == (0, 2 ** 64 - 1)
    assert err_host(err2) == (0, 2 ** 64 - 1)

    def pack_rd_unpack(xs):
        w = [oracle.pack(x, 1) for x in xs]
        o, e = oracle.rd(w, 1)
        x, e2 = oracle.unpack(o[0], 4)
        return w, o, x, int(e[0]) + int(e2[0])

    note("payload full size: compare every word and element with the oracle")
    bad = []
    for a, b in blocks(n, FULL_BLOCK):
        wa, wb = a // 2, b // 2
        parts = pmap_slices(pack_rd_unpack, [down16_range(x, a, b) for x in ins], b - a)
        want_w = [np.concatenate([p[0][r] for p in parts]) for r in range(P)]
        want_o = [np.concatenate([p[1][r] for p in parts]) for r in range(P)]
        want_x = np.concatenate([p[2] for p in parts])
        assert sum(p[3] for p in parts) == 0
        for r in range(P):
            for name, got, want in ((f"pack[{r}]", down64_range(words[r], wa, wb), want_w[r]),
                                    (f"rd fused[{r}]", down64_range(rdo[r], wa, wb), want_o[r]),
                                    (f"rd staged[{r}]", down64_range(rds[r], wa, wb), want_o[r]),
                                    (f"unpack[{r}]", down16_range(xo[r], a, b), want_x)):
                cnt, first = first_mismatch(got, want)
                if cnt:
                    bad.append((name, (wa if name[0] != "u" else a) + first, cnt))
    assert not bad, f"payload path: mismatches (output, first index, count in block) {bad[:8]}"
    record_property("words_compared", 3 * P * W)
    record_property("elements_compared", P * n)
    print(f"[gpu] payload full size: {3 * P} payload outputs x {W} words and {P} x {n} elements equal the oracle")
    del ins, words, rdo, rds, xo
    torch.cuda.empty_cache()


# ------------------------------------------------------------ reordered variants (tolerance)

def _f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _within(got_bits, ref_bits, xs, floor_coef):
    """max relative error 2^-7 (one bf16 ulp) per element, with an absolute
    floor floor_coef * sum_p |x_p| for elements whose exact sum cancels."""
    a, b = _f64(got_bits), _f64(ref_bits)
    absum = sum(np.abs(_f64(x)) for x in xs)
    rel = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b))
    floor = floor_coef * absum
    ok = np.abs(a - b) <= np.maximum(rel, floor)
    by_floor = int(np.count_nonzero((np.abs(a - b) > rel) & ok))
    return bool(ok.all()), by_floor


P8_GAMMA = 7 * 2.0 ** -24 / (1 - 7 * 2.0 ** -24)


@pytest.mark.parametrize("kind", ["normal", "logmag"])
def test_rd_fp32_carry_vs_sequential(kind, record_property):
    """Tree order with binary32 partials vs the sequential schedule: within
    one bf16 ulp, floor 2*gamma_7*sum|x| (two binary32 summation orders).
    On these inputs every element meets the one-ulp bound itself: the count
    judged by the floor is recorded and must stay zero."""
    P, n, seq0 = 8, 128 * HIDDEN, 3
    xs = synth.rank_buffers(kind, P, n, 3, 71)
    ref = oracle.reduce_seq(xs)
    words = [up64(oracle.pack(x, seq0)) for x in xs]
    out = [torch.empty(n // 2, dtype=torch.int64, device=DEV) for _ in range(P)]
    err = new_err()
    note(f"rd fp32-carry vs sequential {kind}")
    tar.ar_rd_schedule(words, out, seq0, err, flags=tar.AR_RD_FP32_CARRY)
    x = empty16(n)
    tar.ar_unpack_fused(out[0], x, seq0 + 3, err)
    torch.cuda.synchronize()
    assert err_host(err)[0] == 0
    ok, by_floor = _within(down16(x), ref, xs, 2 * P8_GAMMA)
    print(f"[gpu] fp32-carry {kind}: {by_floor} of {n} elements judged by the cancellation floor")
    record_property("judged_by_floor", by_floor)
    assert ok
    assert by_floor == 0


@pytest.mark.parametrize("kind", ["normal", "logmag"])
def test_rd_round_each_step_vs_sequential(kind, record_property):
    """Per-step bf16 rounding vs the sequential schedule: within one bf16 ulp,
    or the absolute floor (4*2^-8 + 2*gamma_7)*sum|x|: three tree levels each
    round partials whose magnitudes sum to at most sum|x|, plus the
    sequential result's own final rounding and binary32 accumulation."""
    P, n, seq0 = 8, 128 * HIDDEN, 5
    xs = synth.rank_buffers(kind, P, n, 3, 72)
    ref = oracle.reduce_seq(xs)
    words = [up64(oracle.pack(x, seq0)) for x in xs]
    out = [torch.empty(n // 2, dtype=torch.int64, device=DEV) for _ in range(P)]
    err = new_err()
    note(f"rd round-each-step vs sequential {kind}")
    tar.ar_rd_schedule(words, out, seq0, err)
    x = empty16(n)
    tar.ar_unpack_fused(out[5], x, seq0 + 3, err)
    torch.cuda.synchronize()
    ok, by_floor = _within(down16(x), ref, xs, 4 * 2.0 ** -8 + 2 * P8_GAMMA)
    print(f"[gpu] round-each-step {kind}: {by_floor} of {n} elements judged by the floor")
    record_property("judged_by_floor", by_floor)
    assert ok
    # per-step rounding is a different schedule: a sizeable share of the
    # elements needs the floor, but far from all of them
    assert by_floor <= n // 4


def test_permuted_ranks_within_tolerance(record_property):
    """The rank order is part of the schedule: permuting the inputs gives a
    reordered sum, within one bf16 ulp of the sequential oracle (floor
    2*gamma_7*sum|x|); integer data is exact in any order.  On these inputs
    every element meets the one-ulp bound itself: the count judged by the
    floor is recorded and must stay zero."""
    P, n = 8, 32 * HIDDEN
    xs = synth.rank_buffers("normal", P, n, 2, 73)
    ref = oracle.reduce_seq(xs)
    g = np.random.default_rng(74)
    for _ in range(3):
        perm = g.permutation(P)
        out = empty16(n)
        note(f"permuted ranks {perm.tolist()}")
        tar.ar_reduce_oneshot([up16(xs[p]) for p in perm], out)
        torch.cuda.synchronize()
        ok, by_floor = _within(down16(out), ref, xs, 2 * P8_GAMMA)
        record_property(f"judged_by_floor_{'_'.join(map(str, perm.tolist()))}", by_floor)
        assert ok
        assert by_floor == 0
    ints = synth.rank_buffers("integers", P, n, 2, 75)
    iref = oracle.reduce_seq(ints)
    out = empty16(n)
    tar.ar_reduce_oneshot([up16(ints[p]) for p in g.permutation(P)], out)
    torch.cuda.synchronize()
    check_full(out, iref, "permuted integers")


# ------------------------------------------------------------ HIP graph capture

def test_graph_capture_replays():
    """The hot-path calls (error-record init, one-shot, fused two-stage, pack,
    recursive doubling, unpack) captured in one HIP graph; the graph is
    replayed several times with fresh inputs copied in and eager library
    calls between replays, and every replay is checked against the oracle."""
    P, n = 8, 32 * HIDDEN
    ins = [empty16(n) for _ in range(P)]
    out1 = empty16(n)
    outs = [empty16(n) for _ in range(P)]
    words = [torch.empty(n // 2, dtype=torch.int64, device=DEV) for _ in range(P)]
    rdo = [torch.empty(n // 2, dtype=torch.int64, device=DEV) for _ in range(P)]
    x = empty16(n)
    err = torch.empty(2, dtype=torch.int64, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    note("graph capture")
    with torch.cuda.stream(side):
        # warm the library's one-time initialisation outside the capture
        tar.ar_err_init(err, stream=side)
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            tar.ar_err_init(err, stream=side)
            tar.ar_reduce_oneshot(ins, out1, stream=side)
            tar.ar_reduce_2stage(ins, outs, stream=side)
            for r in range(P):
                tar.ar_pack_fused(ins[r], words[r], 9, stream=side)
            tar.ar_rd_schedule(words, rdo, 9, err, stream=side)
            tar.ar_unpack_fused(rdo[2], x, 12, err, stream=side)
    torch.cuda.synchronize()
    for rep in range(4):
        xs = synth.rank_buffers("normal", P, n, 60, rep)
        for t, h in zip(ins, xs):
            t.copy_(up16(h))
        # eager library work between replays, on the default stream
        scratch_out = empty16(n)
        tar.ar_reduce_oneshot(ins[::-1], scratch_out)
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.reduce_seq(xs)
        check_full(out1, ref, f"graph replay {rep} oneshot")
        for o in outs:
            check_full(o, ref, f"graph replay {rep} 2stage")
        rw, _ = oracle.rd([oracle.pack(v, 9) for v in xs], 9)
        want, _ = oracle.unpack(rw[2], 12)
        check_full(x, want, f"graph replay {rep} rd")
        assert err_host(err) == (0, 2 ** 64 - 1)
        check_full(scratch_out, oracle.reduce_seq(xs[::-1]), "eager between replays")


def test_graph_capture_prepared_calls():
    """Prepared handles (tar.prepare, stream fixed to the capture stream) for
    the decode-size one-shot, fused two-stage with separate outputs and in
    place, captured in one HIP graph; replayed with fresh inputs written into
    the same buffers and eager wrapper calls between replays, every replay
    checked against the oracle."""
    P, n = 8, 16 * HIDDEN + 5
    ins, bufs = [empty16(n) for _ in range(P)], [empty16(n) for _ in range(P)]
    out1, outs = empty16(n), [empty16(n) for _ in range(P)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    hs = [tar.prepare(tar.ar_reduce_oneshot, ins, out1, stream=side),
          tar.prepare(tar.ar_reduce_2stage, ins, outs, stream=side),
          tar.prepare(tar.ar_reduce_2stage, bufs, bufs, stream=side)]
    g = torch.cuda.CUDAGraph()
    note("graph capture of prepared calls")
    with torch.cuda.stream(side):
        for h in hs:                             # the library's one-time initialisation, outside the capture
            h()
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            for h in hs:
                h()
    torch.cuda.synchronize()
    for rep in range(3):
        xs = synth.rank_buffers("normal", P, n, 61, rep)
        for t, b, x in zip(ins, bufs, xs):
            t.copy_(up16(x))
            b.copy_(up16(x))
        between = empty16(n)
        tar.ar_reduce_2stage(ins[::-1], [between] + [empty16(n) for _ in range(P - 1)])
        torch.cuda.synchronize()
        note(f"prepared graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.reduce_seq(xs)
        check_full(out1, ref, f"prepared graph replay {rep} oneshot")
        for r in range(P):
            check_full(outs[r], ref, f"prepared graph replay {rep} 2stage rank {r}")
            check_full(bufs[r], ref, f"prepared graph replay {rep} in place rank {r}")
        check_full(between, oracle.reduce_seq(xs[::-1]), "eager between replays")


def test_graph_capture_replays_other_calls():
    """The remaining entry points captured in one HIP graph: the staged
    two-stage (caller scratch, and the library's static scratch -- the
    no-allocation entry point exists for callers under graph capture),
    staged recursive doubling (mailbox), the waiting unpack on payloads the
    graph itself produced, the two-stream ubatch reduce on the flat and the
    bounded grid and with completion flags (the ubatch streams forked from
    the capture stream and joined back), and the fp8 quantise and reduce.
    Replayed with fresh inputs, cleared outputs and flags, and eager library
    work between replays (including an eager static-scratch call on other
    values, which leaves its own values in the shared array); every replay
    is checked against the oracle."""
    P, rows = 8, 24
    n = rows * HIDDEN
    chunk = 64 * 1024 + 16                     # bytes: chunks end off the row boundaries

    def i64(k):
        return torch.empty(k, dtype=torch.int64, device=DEV)
    ins = [empty16(n) for _ in range(P)]
    st_outs, ub_outs, fl_outs, f8_outs, sa_outs, bd_outs, eg_outs = ([empty16(n) for _ in range(P)]
                                                                     for _ in range(7))
    scratch, xw = empty16(n), empty16(n)
    words, rdo = [i64(n // 2) for _ in range(P)], [i64(n // 2) for _ in range(P)]
    mbox = i64(tar.rd_mailbox_words(P, n))
    nflags = tar.ubatch_chunk_count(rows, HIDDEN, 2, None, chunk)
    done = torch.zeros(nflags, dtype=torch.int32, device=DEV)
    tiles = torch.zeros(nflags, dtype=torch.int32, device=DEV)
    codes = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(P)]
    scales = [torch.empty(tar.fp8_scale_count(n), dtype=torch.uint8, device=DEV) for _ in range(P)]
    err = torch.empty(2, dtype=torch.int64, device=DEV)
    side, s0, s1 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()

    def body():
        tar.ar_err_init(err, stream=side)
        tar.ar_reduce_2stage(ins, st_outs, scratch=scratch, stream=side)
        tar.ar_reduce_2stage_static(ins, sa_outs, stream=side)
        for r in range(P):
            tar.ar_pack_fused(ins[r], words[r], 21, stream=side)
        tar.ar_rd_schedule(words, rdo, 21, err, mailbox=mbox, flags=tar.AR_RD_STAGED, stream=side)
        tar.ar_unpack_fused_wait(rdo[6], xw, 24, err, max_spins=1000, stream=side)
        s0.wait_stream(side)
        s1.wait_stream(side)
        tar.ar_reduce_ubatch(ins, ub_outs, rows, HIDDEN, 2, None, chunk, tar.AR_VARIANT_2STAGE, streams=[s0, s1])
        tar.ar_reduce_ubatch_flags(ins, fl_outs, rows, HIDDEN, done, tiles, 5, 2, None, chunk,
                                   tar.AR_VARIANT_ONESHOT, streams=[s0, s1])
        tar.ar_reduce_ubatch(ins, bd_outs, rows, HIDDEN, 2, None, chunk,
                             tar.AR_VARIANT_2STAGE | tar.AR_UBATCH_BOUNDED, streams=[s0, s1])
        side.wait_stream(s0)
        side.wait_stream(s1)
        tar.ar_quantize_fp8(ins, codes, scales, stream=side)
        tar.ar_reduce_fp8(codes, scales, f8_outs, stream=side)

    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    note("graph capture of the remaining entry points")
    with torch.cuda.stream(side):
        body()                                 # eager once: one-time initialisation outside the capture
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            body()
    torch.cuda.synchronize()
    for rep in range(3):
        xs = synth.rank_buffers("normal", P, n, 61, rep)
        for t, h in zip(ins, xs):
            t.copy_(up16(h))
        for t in st_outs + ub_outs + fl_outs + f8_outs + sa_outs + bd_outs + [scratch, xw]:
            t.zero_()
        done.zero_()
        scratch_out = empty16(n)
        tar.ar_reduce_oneshot(ins[::-1], scratch_out)
        tar.ar_reduce_2stage_static(ins[::-1], eg_outs)
        torch.cuda.synchronize()
        note(f"graph replay {rep} of the remaining entry points")
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.reduce_seq(xs)
        check_full(scratch, ref, f"replay {rep} staged scratch")
        for o in st_outs + ub_outs + sa_outs + bd_outs:
            check_full(o, ref, f"replay {rep} staged two-stage / ubatch")
        check_full(fl_outs[0], ref, f"replay {rep} flagged ubatch")
        assert bool((done == 5).all()) and not bool(tiles.any()), f"replay {rep}: chunk flags or counters"
        rw, _ = oracle.rd([oracle.pack(v, 21) for v in xs], 21)
        for o, w in zip(rdo, rw):
            assert np.array_equal(down64(o), w), f"replay {rep}: staged RD payload"
        want, _ = oracle.unpack(rw[6], 24)
        check_full(xw, want, f"replay {rep} waiting unpack")
        assert err_host(err) == (0, 2 ** 64 - 1)
        q = [oracle.quant_fp8(v) for v in xs]
        for t, (c, sc), t2 in zip(codes, q, scales):
            assert np.array_equal(t.cpu().numpy(), c) and np.array_equal(t2.cpu().numpy(), sc), \
                f"replay {rep}: fp8 codes or scales"
        f8 = oracle.reduce_fp8([c for c, _ in q], [sc for _, sc in q])
        for o in f8_outs:
            check_full(o, f8, f"replay {rep} fp8 reduce")
        check_full(scratch_out, oracle.reduce_seq(xs[::-1]), "eager between replays")
        for o in eg_outs:
            check_full(o, oracle.reduce_seq(xs[::-1]), "eager static-scratch call between replays")
