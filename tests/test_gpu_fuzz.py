"""Seeded random cases across every entry point against the oracle.

Each case draws the rank count, the element count (tiny, ragged, or a few
tiles), the value mix (normal, log-uniform, integers, or specials mixed in),
and the operation's own knobs (chunk size, ubatch split and grid, sequence
number, output count), then compares every output with the oracle bit for
bit.  The reduce family runs the one-shot, the fused (separate outputs and
in place), staged and static-scratch two-stage, and the ubatch reduce on the
flat or the bounded grid; the payload family ends with the plain or the
waiting unpack.  The
seed of a failing case is in the assertion message.  AR_FUZZ_SEEDS=<k> in
the environment runs k seeds per family, and AR_FUZZ_SEED0=<s> starts them
at s instead of 0 (a soak over cases the default run never draws).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_amd as tar
from tensor_all_reduce_amd import synth
from gpu_util import DEV, note, up16, down16, up64, down64, empty16, new_err, err_host

pytestmark = pytest.mark.gpu

# seeds per family; AR_FUZZ_SEEDS=<k> runs k seeds of every family instead
# (a longer soak), starting at AR_FUZZ_SEED0 (default 0, where the default
# range starts)
_K = os.environ.get("AR_FUZZ_SEEDS")
N_REDUCE, N_PAYLOAD, N_FP8 = (int(_K),) * 3 if _K else (80, 80, 60)
S0 = int(os.environ.get("AR_FUZZ_SEED0", "0"))

SPECIALS = np.array([0x7FC0, 0xFFC1, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0xFF7F, 0x0080],
                    dtype=np.uint16)


def draw(rng, P, n, seed):
    kind = rng.choice(["normal", "logmag", "integers", "specials"])
    xs = synth.rank_buffers("normal" if kind == "specials" else kind, P, n, 990, seed)
    if kind == "specials" and n:
        for x in xs:
            k = int(rng.integers(1, max(2, n // 8)))
            x[rng.integers(0, n, size=k)] = rng.choice(SPECIALS, size=k)
    return xs, kind


def size(rng):
    r = rng.random()
    if r < 0.25:
        return int(rng.integers(0, 40))
    if r < 0.75:
        return int(rng.integers(40, 5000))
    return int(rng.integers(5000, 70000))


def eq(got, want, msg):
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{msg}: {bad.size} mismatches, first at {bad[0]}: got {got[bad[0]]:#x} want {want[bad[0]]:#x}"


@pytest.mark.parametrize("seed", range(S0, S0 + N_REDUCE))
def test_fuzz_reduce_family(seed):
    rng = np.random.default_rng([991, seed])
    P = int(rng.integers(1, 9))
    n = size(rng)
    xs, kind = draw(rng, P, n, seed)
    tag = f"seed {seed}: P={P} n={n} {kind}"
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) if n else empty16(1) for x in xs]     # n = 0: a real (unused) pointer
    note(f"fuzz reduce {tag}")
    out = empty16(max(n, 1))
    tar.ar_reduce_oneshot(ins, out, n=n)
    outs = [empty16(max(n, 1)) for _ in range(P)]
    tar.ar_reduce_2stage(ins, outs, n=n)
    scratch = empty16(max(n, 1))
    outs2 = [empty16(max(n, 1)) for _ in range(P)]
    tar.ar_reduce_2stage(ins, outs2, scratch=scratch, n=n)
    outs3 = [empty16(max(n, 1)) for _ in range(P)]
    tar.ar_reduce_2stage_static(ins, outs3, n=n)
    bufs = [up16(x) if n else empty16(1) for x in xs]    # fused, in place
    tar.ar_reduce_2stage(bufs, bufs, n=n)
    torch.cuda.synchronize()
    eq(down16(out)[:n], ref, f"{tag} oneshot")
    for o in outs + outs2 + outs3 + bufs:
        eq(down16(o)[:n], ref, f"{tag} 2stage")
    # ubatch: a random factorisation of n into rows x hidden and a random split
    if n:
        divs = [d for d in range(1, min(n, 64) + 1) if n % d == 0]
        rows = int(rng.choice(divs))
        hidden = n // rows
        nub = int(rng.integers(1, min(rows, 4) + 1))
        cuts = np.sort(rng.choice(np.arange(1, rows), size=nub - 1, replace=False)) if nub > 1 else []
        split = np.diff(np.concatenate([[0], cuts, [rows]])).astype(int).tolist()
        chunk = 16 * int(rng.integers(1, 300))
        variant = int(rng.integers(0, 2))
        bounded = bool(rng.integers(0, 2))
        uouts = [empty16(n) for _ in range(P)]
        note(f"fuzz ubatch {tag} rows={rows} split={split} chunk={chunk} variant={variant} bounded={bounded}")
        tar.ar_reduce_ubatch(ins, uouts, rows, hidden, nub, split, chunk,
                             variant | (tar.AR_UBATCH_BOUNDED if bounded else 0))
        torch.cuda.synchronize()
        for o in (uouts if variant == tar.AR_VARIANT_2STAGE else uouts[:1]):
            eq(down16(o), ref, f"{tag} ubatch")


@pytest.mark.parametrize("seed", range(S0, S0 + N_PAYLOAD))
def test_fuzz_payload_family(seed):
    rng = np.random.default_rng([992, seed])
    P = int(rng.choice([2, 4, 8]))
    n = 2 * (size(rng) // 2)
    xs, kind = draw(rng, P, n, seed)
    seq0 = int(rng.choice([0, 1, 0x7FFFFFFF, 0xFFFFFFFE, 0xFFFFFFFF, int(rng.integers(0, 2 ** 32))]))
    staged = bool(rng.integers(0, 2))
    carry = (not staged) and bool(rng.integers(0, 2))
    wait = bool(rng.integers(0, 2))
    tag = f"seed {seed}: P={P} n={n} {kind} seq0={seq0:#x} staged={staged} carry={carry} wait={wait}"
    note(f"fuzz payload {tag}")
    W = n // 2
    words = [torch.empty(max(W, 1), dtype=torch.int64, device=DEV) for _ in range(P)]
    for p in range(P):
        tar.ar_pack_fused(up16(xs[p]) if n else empty16(1), words[p], seq0, n=n)
    rdo = [torch.empty(max(W, 1), dtype=torch.int64, device=DEV) for _ in range(P)]
    err = new_err()
    mbox = torch.empty(max(tar.rd_mailbox_words(P, n), 1), dtype=torch.int64, device=DEV) if staged else None
    flags = (tar.AR_RD_STAGED if staged else 0) | (tar.AR_RD_FP32_CARRY if carry else 0)
    tar.ar_rd_schedule(words, rdo, seq0, err, mailbox=mbox, flags=flags, n=n)
    L = {2: 1, 4: 2, 8: 3}[P]
    out = empty16(max(n, 1))
    if wait:   # the payload is already written: the waiting unpack must take every word at once
        tar.ar_unpack_fused_wait(rdo[P - 1], out, (seq0 + L) & 0xFFFFFFFF, err, n=n)
    else:
        tar.ar_unpack_fused(rdo[P - 1], out, (seq0 + L) & 0xFFFFFFFF, err, n=n)
    torch.cuda.synchronize()
    ow = [oracle.pack(x, seq0) for x in xs]
    for p in range(P):
        eq(down64(words[p])[:W], ow[p], f"{tag} pack")
    want, werr = oracle.rd(ow, seq0, carry)
    for p in range(P):
        eq(down64(rdo[p])[:W], want[p], f"{tag} rd")
    assert err_host(err) == (0, 2 ** 64 - 1), tag
    eq(down16(out)[:n], oracle.unpack(want[P - 1], (seq0 + L) & 0xFFFFFFFF)[0], f"{tag} unpack")


@pytest.mark.parametrize("seed", range(S0, S0 + N_FP8))
def test_fuzz_fp8_family(seed):
    rng = np.random.default_rng([993, seed])
    P = int(rng.integers(1, 9))
    n = size(rng)
    xs, kind = draw(rng, P, n, seed)
    tag = f"seed {seed}: P={P} n={n} {kind}"
    note(f"fuzz fp8 {tag}")
    nb = tar.fp8_scale_count(n)
    codes = [torch.empty(max(n, 16), dtype=torch.uint8, device=DEV) for _ in range(P)]
    scales = [torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV) for _ in range(P)]
    tar.ar_quantize_fp8([up16(x) if n else empty16(1) for x in xs], codes, scales, n=n)
    nout = P if rng.integers(0, 2) else 1
    outs = [empty16(max(n, 1)) for _ in range(nout)]
    tar.ar_reduce_fp8(codes, scales, outs, n=n)
    torch.cuda.synchronize()
    q = [oracle.quant_fp8(x) for x in xs]
    for p in range(P):
        eq(codes[p].cpu().numpy()[:n], q[p][0], f"{tag} codes")
        eq(scales[p].cpu().numpy()[:nb], q[p][1], f"{tag} scales")
    want = oracle.reduce_fp8([c for c, _ in q], [s for _, s in q])
    for o in outs:
        eq(down16(o)[:n], want, f"{tag} reduce")
