"""Every launch-shape variant of every kernel against the oracle.

The library picks one shape per kernel kind (block size, groups per lane,
non-temporal loads / stores, workgroups per CU); each choice is a different
kernel instantiation or grid.  Here each kind is run under a grid of shapes
on ragged sizes (tails inside a 16-byte group and inside a tile) and every
result is compared with the oracle, bit for bit; the default shape is
restored afterwards (the fused two-stage also in place, which at small sizes
takes its own compact kernel).  The one-shot, fused two-stage, fused RD, staged RD,
pack and unpack calls pick their small-message kind at n <= AR_SMALL_ELEMS
and their large-message kind above it, so those run at one size on each side
of the threshold.
"""
import functools
import itertools

import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_amd as tar
from tensor_all_reduce_amd import synth
from gpu_util import DEV, note, up16, down16, up64, down64, empty16, new_err, err_host

pytestmark = pytest.mark.gpu

SHAPES = [(b, v, ntl, nts, wg) for b, v, ntl, nts, wg in
          itertools.product((64, 256), (1, 2), (0, 1), (0, 1), (0, 3))]
# 128-lane workgroups (each a compile-time block size of the small-message and
# staged kernels) with the two write-through store policies
SHAPES += [(128, 1, 0, 2, 0), (128, 1, 1, 3, 0), (128, 2, 1, 2, 3), (128, 2, 0, 3, 0)]
P = 8
N = 5 * 4096 + 22          # even; not a multiple of 8 or 16
ROWS, HIDDEN = 11, 1862    # 20482 elements, odd row count and a hidden size not a multiple of 8

NL = tar.AR_SMALL_ELEMS + 4096 + 22   # above the small-message threshold; not a multiple of 8

XS = synth.rank_buffers("logmag", P, N, 900)
REF = oracle.reduce_seq(XS)


@functools.lru_cache(maxsize=1)
def large():
    """Inputs above the threshold and their oracle results (built on first use,
    not at collection)."""
    xl = synth.rank_buffers("logmag", P, NL, 901)
    words = [oracle.pack(x, 9) for x in xl]         # NL / 2 words: odd, so RD's one-lane tail runs
    return xl, oracle.reduce_seq(xl), words, {carry: oracle.rd(words, 9, carry) for carry in (False, True)}


def with_shape(kinds, shape, fn):
    kinds = kinds if isinstance(kinds, (tuple, list)) else (kinds,)
    before = [tar.ar_get_launch_shape(k) for k in kinds]
    for k in kinds:
        tar.ar_set_launch_shape(k, *shape)
    try:
        fn()
        torch.cuda.synchronize()
    finally:
        for k, b in zip(kinds, before):
            tar.ar_set_launch_shape(k, *b)


ONESHOT_KINDS = (tar.AR_KERNEL_ONESHOT, tar.AR_KERNEL_ONESHOT_SMALL)
TWOSTAGE_KINDS = (tar.AR_KERNEL_2STAGE, tar.AR_KERNEL_2STAGE_SMALL, tar.AR_KERNEL_2STAGE_INPLACE_SMALL)
RD_KINDS = (tar.AR_KERNEL_RD, tar.AR_KERNEL_RD_SMALL)
RDSTEP_KINDS = (tar.AR_KERNEL_RDSTEP, tar.AR_KERNEL_RDSTEP_SMALL)
PACK_KINDS = (tar.AR_KERNEL_PACK, tar.AR_KERNEL_PACK_SMALL)
UNPACK_KINDS = (tar.AR_KERNEL_UNPACK, tar.AR_KERNEL_UNPACK_SMALL)


def eq(got, want, what):
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[0]}"


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}v{}l{}s{}w{}".format(*s))
def test_reduce_kinds(shape):
    xl, refl = large()[:2]
    for xs, ref, n in ((XS, REF, N), (xl, refl, NL)):
        ins = [up16(x) for x in xs]
        note(f"shape {shape}: oneshot n={n}")
        out = empty16(n)
        with_shape(ONESHOT_KINDS, shape, lambda: tar.ar_reduce_oneshot(ins, out))
        eq(down16(out), ref, f"oneshot n={n}")
        note(f"shape {shape}: 2stage fused n={n}")
        outs = [empty16(n) for _ in range(P)]
        with_shape(TWOSTAGE_KINDS, shape, lambda: tar.ar_reduce_2stage(ins, outs))
        for o in outs:
            eq(down16(o), ref, f"2stage n={n}")
        note(f"shape {shape}: 2stage fused in place n={n}")
        bufs = [up16(x) for x in xs]
        with_shape(TWOSTAGE_KINDS, shape, lambda: tar.ar_reduce_2stage(bufs, bufs))
        for b in bufs:
            eq(down16(b), ref, f"2stage in place n={n}")
    ins = [up16(x) for x in XS]
    note(f"shape {shape}: 2stage staged (rs, then ag)")
    for kind in (tar.AR_KERNEL_RS, tar.AR_KERNEL_AG):
        outs = [empty16(N) for _ in range(P)]
        scratch = empty16(N)
        with_shape(kind, shape, lambda: tar.ar_reduce_2stage(ins, outs, scratch=scratch))
        for o in outs:
            eq(down16(o), REF, f"staged kind {kind}")
        eq(down16(scratch), REF, "staged scratch")
    note(f"shape {shape}: ubatch and flagged ubatch")
    ub = [4, 7]
    xs = [x[: ROWS * HIDDEN] for x in XS]
    ref = oracle.reduce_seq(xs)
    ui = [up16(x) for x in xs]
    for kind in (tar.AR_KERNEL_UBATCH, tar.AR_KERNEL_ONESHOT):
        outs = [empty16(ROWS * HIDDEN) for _ in range(P)]
        variant = tar.AR_VARIANT_2STAGE if kind == tar.AR_KERNEL_UBATCH else tar.AR_VARIANT_ONESHOT
        with_shape(kind, shape, lambda: tar.ar_reduce_ubatch(ui, outs, ROWS, HIDDEN, 2, ub, 4096 + 16, variant))
        for o in (outs if variant == tar.AR_VARIANT_2STAGE else outs[:1]):
            eq(down16(o), ref, f"ubatch kind {kind}")
    nflags = tar.ubatch_chunk_count(ROWS, HIDDEN, 2, ub, 4096 + 16)
    done = torch.zeros(nflags, dtype=torch.int32, device=DEV)
    tiles = torch.zeros(nflags, dtype=torch.int32, device=DEV)
    outs = [empty16(ROWS * HIDDEN) for _ in range(P)]
    with_shape(tar.AR_KERNEL_UBATCH_FLAGS, shape,
               lambda: tar.ar_reduce_ubatch_flags(ui, outs, ROWS, HIDDEN, done, tiles, 7, 2, ub, 4096 + 16,
                                                  tar.AR_VARIANT_2STAGE))
    for o in outs:
        eq(down16(o), ref, "flagged ubatch")
    assert np.all(done.cpu().numpy() == 7) and not tiles.cpu().numpy().any()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}v{}l{}s{}w{}".format(*s))
def test_payload_kinds(shape):
    n = N - 4                                  # odd word count (10249): the one-lane tail of RD
    xs = [x[:n] for x in XS]
    words_ref = [oracle.pack(x, 9) for x in xs]
    ins = [up16(x) for x in xs]
    note(f"shape {shape}: pack")
    words = [torch.empty(n // 2, dtype=torch.int64, device=DEV) for _ in range(P)]

    def pack_all():
        for i in range(P):
            tar.ar_pack_fused(ins[i], words[i], 9)
    with_shape(PACK_KINDS, shape, pack_all)
    for w, r in zip(words, words_ref):
        eq(down64(w), r, "pack")
    for kind, flags, carry in ((RD_KINDS, 0, False), (RD_KINDS, tar.AR_RD_FP32_CARRY, True),
                               (RDSTEP_KINDS, tar.AR_RD_STAGED, False)):
        note(f"shape {shape}: rd kind {kind} flags {flags}")
        outs = [torch.empty(n // 2, dtype=torch.int64, device=DEV) for _ in range(P)]
        mbox = torch.empty(tar.rd_mailbox_words(P, n), dtype=torch.int64, device=DEV) if flags & tar.AR_RD_STAGED else None
        err = new_err()
        with_shape(kind, shape, lambda: tar.ar_rd_schedule(words, outs, 9, err, mailbox=mbox, flags=flags))
        want, werr = oracle.rd(words_ref, 9, carry)
        for o, w in zip(outs, want):
            eq(down64(o), w, f"rd kind {kind}")
        assert err_host(err) == (int(werr[0]), int(werr[1]))
    note(f"shape {shape}: unpack and waiting unpack")
    for kind in (UNPACK_KINDS, tar.AR_KERNEL_UNPACK_WAIT):
        out = empty16(n)
        err = new_err()
        if kind == UNPACK_KINDS:
            fn = lambda: tar.ar_unpack_fused(words[2], out, 9, err)
        else:
            fn = lambda: tar.ar_unpack_fused_wait(words[2], out, 9, err, max_spins=100)
        with_shape(kind, shape, fn)
        eq(down16(out), xs[2], f"unpack kind {kind}")
        assert err_host(err) == (0, 2 ** 64 - 1)
    note(f"shape {shape}: fused and staged rd above the small-message threshold (n={NL})")
    _, _, words_ref_l, rd_l = large()
    words_l = [up64(w) for w in words_ref_l]
    mbox_l = torch.empty(tar.rd_mailbox_words(P, NL), dtype=torch.int64, device=DEV)
    for kinds, flags, carry in ((RD_KINDS, 0, False), (RD_KINDS, tar.AR_RD_FP32_CARRY, True),
                                (RDSTEP_KINDS, tar.AR_RD_STAGED, False)):
        outs = [torch.empty(NL // 2, dtype=torch.int64, device=DEV) for _ in range(P)]
        err = new_err()
        mb = mbox_l if flags & tar.AR_RD_STAGED else None
        with_shape(kinds, shape, lambda: tar.ar_rd_schedule(words_l, outs, 9, err, mailbox=mb, flags=flags))
        want, werr = rd_l[carry]
        for o, w in zip(outs, want):
            eq(down64(o), w, f"rd n={NL} flags={flags}")
        assert err_host(err) == (int(werr[0]), int(werr[1]))
    note(f"shape {shape}: pack and unpack above the small-message threshold (n={NL})")
    xl = large()[0]
    xin = up16(xl[3])
    wl = torch.empty(NL // 2, dtype=torch.int64, device=DEV)
    with_shape(PACK_KINDS, shape, lambda: tar.ar_pack_fused(xin, wl, 9))
    eq(down64(wl), words_ref_l[3], f"pack n={NL}")
    out = empty16(NL)
    err = new_err()
    with_shape(UNPACK_KINDS, shape, lambda: tar.ar_unpack_fused(words_l[5], out, 9, err))
    eq(down16(out), xl[5], f"unpack n={NL}")
    assert err_host(err) == (0, 2 ** 64 - 1)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}v{}l{}s{}w{}".format(*s))
def test_fp8_kinds(shape):
    q = [oracle.quant_fp8(x) for x in XS]
    want = oracle.reduce_fp8([c for c, _ in q], [s for _, s in q])
    ins = [up16(x) for x in XS]
    note(f"shape {shape}: fp8 quantise")
    codes = [torch.empty(N, dtype=torch.uint8, device=DEV) for _ in range(P)]
    scales = [torch.empty(tar.fp8_scale_count(N), dtype=torch.uint8, device=DEV) for _ in range(P)]
    with_shape(tar.AR_KERNEL_QUANT_FP8, shape, lambda: tar.ar_quantize_fp8(ins, codes, scales))
    for p in range(P):
        eq(codes[p].cpu().numpy(), q[p][0], "fp8 codes")
        eq(scales[p].cpu().numpy(), q[p][1], "fp8 scales")
    for kind, nout in ((tar.AR_KERNEL_REDUCE_FP8, 1), (tar.AR_KERNEL_REDUCE_FP8_ALL, P)):
        note(f"shape {shape}: fp8 reduce -> {nout}")
        outs = [empty16(N) for _ in range(nout)]
        with_shape(kind, shape, lambda: tar.ar_reduce_fp8(codes, scales, outs))
        for o in outs:
            eq(down16(o), want, f"fp8 reduce -> {nout}")
