"""The entry point that allocates nothing: ar_reduce_2stage_static.

It runs the staged two-stage kernels with the library's static scratch array
instead of a caller's workspace.  Checked through the C-ABI against the
existing staged entry point (ar_reduce_2stage with a caller scratch buffer),
bit for bit, on two calls in a row -- the first at the largest size the
array takes, the second smaller and ragged, so the second call runs on a
scratch array that still holds the first call's values -- and both against
the oracle.  Sizes beyond the array are rejected before any launch.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_amd as tar
from tensor_all_reduce_amd import synth
from gpu_util import DEV, note, up16, down16, empty16, bits16

pytestmark = pytest.mark.gpu


def _staged_pair(xs, P, n, what):
    """Run the static entry point and the existing staged one on the same
    inputs; return both results on the host."""
    ins = [up16(x) for x in xs]
    out_static = [torch.full((n,), 0x5A5A, dtype=torch.int16, device=DEV) for _ in range(P)]
    out_staged = [empty16(n) for _ in range(P)]
    scratch = empty16(n)
    note(f"static scratch: {what}, P={P}, n={n}")
    tar.ar_reduce_2stage_static(ins, out_static)
    tar.ar_reduce_2stage(ins, out_staged, scratch=scratch)
    torch.cuda.synchronize()
    return [down16(o) for o in out_static], [down16(o) for o in out_staged]


def test_static_scratch_matches_staged_two_calls():
    P = 8
    n1 = tar.AR_STATIC_SCRATCH_ELEMS            # the largest size the array takes
    xs1 = synth.rank_buffers("normal", P, n1, 4, 901)
    got1, want1 = _staged_pair(xs1, P, n1, "call 1 (maximum size)")
    ref1 = oracle.reduce_seq(xs1)
    for r in range(P):
        assert np.array_equal(got1[r], want1[r]), f"call 1 rank {r} differs from the staged entry point"
        assert np.array_equal(got1[r], ref1), f"call 1 rank {r} differs from the oracle"
    del xs1, got1, want1, ref1

    n2 = 3 * 8192 + 13                            # smaller, ragged: the array still holds call 1's values
    xs2 = synth.rank_buffers("logmag", P, n2, 4, 902)
    got2, want2 = _staged_pair(xs2, P, n2, "call 2 (smaller, ragged)")
    ref2 = oracle.reduce_seq(xs2)
    for r in range(P):
        assert np.array_equal(got2[r], want2[r]), f"call 2 rank {r} differs from the staged entry point"
        assert np.array_equal(got2[r], ref2), f"call 2 rank {r} differs from the oracle"


def test_static_scratch_other_rank_counts_and_in_place():
    for P, n in ((3, 1000 + 5), (2, 8)):
        xs = synth.rank_buffers("normal", P, n, 4, 903 + P)
        got, want = _staged_pair(xs, P, n, "rank count")
        ref = oracle.reduce_seq(xs)
        for r in range(P):
            assert np.array_equal(got[r], want[r]) and np.array_equal(got[r], ref)
    # in place: every output is its own input
    P, n = 4, 5 * 8192 + 3
    xs = synth.rank_buffers("normal", P, n, 4, 910)
    bufs = [up16(x) for x in xs]
    note("static scratch: in place")
    tar.ar_reduce_2stage_static(bufs, bufs)
    torch.cuda.synchronize()
    ref = oracle.reduce_seq(xs)
    for b in bufs:
        assert np.array_equal(down16(b), ref)


def test_static_scratch_rejects_oversize():
    P, n = 2, tar.AR_STATIC_SCRATCH_ELEMS + 8
    ins = [empty16(n) for _ in range(P)]
    outs = [torch.full((n,), 0x1234, dtype=torch.int16, device=DEV) for _ in range(P)]
    with pytest.raises(tar.ARError) as e:
        tar.ar_reduce_2stage_static(ins, outs)
    assert e.value.code == tar.AR_ERR_SIZE
    torch.cuda.synchronize()
    for o in outs:                                # nothing was queued
        assert bool((bits16(o) == 0x1234).all())


def test_static_scratch_leaves_device_memory_unchanged():
    """After a first round of calls (which loads the kernels and lets the HIP
    runtime size its own launch resources), a second identical round at
    several sizes leaves the device's free memory exactly as it was: the
    scratch is the library's static array, and nothing is allocated per call."""
    P = 8
    sizes = (tar.AR_STATIC_SCRATCH_ELEMS, 3 * 8192 + 5, 64)
    bufs = {n: ([torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)],
                [empty16(n) for _ in range(P)]) for n in sizes}
    note("static scratch: device memory before and after")

    def round_of_calls():
        for _ in range(3):
            for n in sizes:
                tar.ar_reduce_2stage_static(*bufs[n])
        torch.cuda.synchronize()

    round_of_calls()
    free0, _ = torch.cuda.mem_get_info()
    round_of_calls()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, f"device free memory changed by {free0 - free1} bytes"
    for o in bufs[sizes[0]][1]:
        assert bool((bits16(o) == 0).all())
