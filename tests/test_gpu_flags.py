"""Per-chunk completion flags of the chunked ubatch reduce
(ar_reduce_ubatch_flags), with a consumer kernel that waits on them.

Every wait is bounded (max_spins); timeouts are forced from the host by
waiting for an epoch that is never published.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_amd as tar
from tensor_all_reduce_amd import synth
from gpu_util import DEV, note, up16, down16, empty16

pytestmark = pytest.mark.gpu


def bench_lib():
    L = ctypes.CDLL(os.path.join(os.path.dirname(tar.lib_path), "libarbench.so"))
    vp = ctypes.c_void_p
    L.arb_consume_chunks.restype = ctypes.c_int
    L.arb_consume_chunks.argtypes = [vp, ctypes.c_uint32, vp, vp, ctypes.c_size_t, ctypes.c_size_t,
                                     ctypes.c_uint32, ctypes.c_uint32, vp, ctypes.c_int, vp,
                                     ctypes.c_int, vp]
    return L


def u32(n):
    return torch.zeros(n, dtype=torch.int32, device=DEV)


def check(got, want, what):
    g = down16(got)
    bad = np.nonzero(g != want)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[0]}"


def test_flags_set_and_counters_return_to_zero():
    """After each call every chunk flag holds that call's epoch and every tile
    counter is zero again; outputs equal the oracle; the arrays are reused
    across calls without re-initialisation."""
    P, rows, hidden, chunk = 8, 96, 1024, 65536
    n = rows * hidden
    xs = synth.rank_buffers("normal", P, n, 90)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    outs = [empty16(n) for _ in range(P)]
    nchunks = tar.ubatch_chunk_count(rows, hidden, 2, [40, 56], chunk)
    done, tiles = u32(nchunks + 3), u32(nchunks + 3)
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    for epoch in (1, 2, 0x7FFFFFFF):
        for st in s:
            st.wait_stream(torch.cuda.current_stream())
        note(f"flags epoch {epoch}")
        tar.ar_reduce_ubatch_flags(ins, outs, rows, hidden, done, tiles, epoch, 2, [40, 56], chunk,
                                   tar.AR_VARIANT_2STAGE, s)
        torch.cuda.synchronize()
        d = done.cpu().numpy()
        assert np.all(d[:nchunks] == epoch) and np.all(d[nchunks:] == 0)
        assert not tiles.cpu().numpy().any()
        for o in outs:
            check(o, ref, f"epoch {epoch}")


def test_flags_with_the_one_shot_variant():
    """The one-shot variant publishes the same flags; only outs[0] is written
    (the other outputs keep their sentinel)."""
    P, rows, hidden, chunk = 5, 40, 2048 + 8, 4096 + 32
    n = rows * hidden
    xs = synth.rank_buffers("logmag", P, n, 93)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    outs = [torch.full((n,), 0x2222, dtype=torch.int16, device=DEV) for _ in range(P)]
    nchunks = tar.ubatch_chunk_count(rows, hidden, 3, [13, 14, 13], chunk)
    done, tiles = u32(nchunks), u32(nchunks)
    note("flags, one-shot variant")
    tar.ar_reduce_ubatch_flags(ins, outs, rows, hidden, done, tiles, 11, 3, [13, 14, 13], chunk,
                               tar.AR_VARIANT_ONESHOT)
    torch.cuda.synchronize()
    assert np.all(done.cpu().numpy() == 11) and not tiles.cpu().numpy().any()
    check(outs[0], ref, "one-shot flagged")
    for o in outs[1:]:
        assert np.all(down16(o) == 0x2222)


def test_consumer_follows_flags():
    """The producer (flagged reduce) is queued first on one stream, the
    consumer right after on another; the consumer copies each chunk of one
    output as soon as its flag shows the epoch.  Outputs start as a sentinel,
    so a chunk read before it was complete would show up in the copy."""
    P, rows, hidden = 8, 1024, 8192
    n = rows * hidden
    chunk = 1 << 20
    xs = synth.rank_buffers("logmag", P, n, 91)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    outs = [torch.full((n,), 0x5A5A, dtype=torch.int16, device=DEV) for _ in range(P)]
    dst = torch.full((n,), 0x1111, dtype=torch.int16, device=DEV)
    nchunks = tar.ubatch_chunk_count(rows, hidden, 1, None, chunk)
    done, tiles = u32(nchunks), u32(nchunks)
    timeouts = u32(1)
    B = bench_lib()
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    note("consumer follows flags")
    tar.ar_reduce_ubatch_flags(ins, outs, rows, hidden, done, tiles, 5, 1, None, chunk,
                               tar.AR_VARIANT_2STAGE, [prod])
    rc = B.arb_consume_chunks(done.data_ptr(), 5, outs[3].data_ptr(), dst.data_ptr(), n, chunk // 2, 0,
                              1 << 22, timeouts.data_ptr(), 0, None, 512, cons.cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert int(timeouts.item()) == 0
    check(dst, ref, "consumer copy")
    for o in outs:
        check(o, ref, "flagged outputs")


def test_consumer_over_many_epochs_reuses_the_arrays():
    """Twelve producer -> consumer rounds on one pair of flag and counter
    arrays, never re-zeroed: each round's flags carry its own epoch and the
    counters must be back at zero for the next.  Inputs alternate between
    two data sets and the watched output is reset to a sentinel before every
    round, so a chunk taken on a stale flag, or read before it was complete,
    would show up in the copy."""
    P, rows, hidden = 8, 512, 8192
    n = rows * hidden
    chunk = (1 << 20) - 4096 + 16                  # chunks that do not divide the rows evenly
    sets = []
    for seed in (93, 94):
        xs = synth.rank_buffers("logmag", P, n, seed)
        sets.append(([up16(x) for x in xs], oracle.reduce_seq(xs)))
    outs = [empty16(n) for _ in range(P)]
    dst = empty16(n)
    nchunks = tar.ubatch_chunk_count(rows, hidden, 1, None, chunk)   # one ubatch: chunk g starts at g * chunk
    done, tiles = u32(nchunks), u32(nchunks)
    timeouts = u32(1)
    B = bench_lib()
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    for epoch in range(1, 13):
        ins, ref = sets[epoch % 2]
        outs[5].fill_(0x5A5A)
        dst.fill_(0x1111)
        prod.wait_stream(torch.cuda.current_stream())
        cons.wait_stream(torch.cuda.current_stream())
        note(f"flags epoch {epoch} of 12")
        tar.ar_reduce_ubatch_flags(ins, outs, rows, hidden, done, tiles, epoch, 1, None, chunk,
                                   tar.AR_VARIANT_2STAGE, [prod])
        rc = B.arb_consume_chunks(done.data_ptr(), epoch, outs[5].data_ptr(), dst.data_ptr(), n, chunk // 2, 0,
                                  1 << 22, timeouts.data_ptr(), 0, None, 256, cons.cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        assert int(timeouts.item()) == 0, f"epoch {epoch}"
        check(dst, ref, f"consumer copy, epoch {epoch}")
        for o in outs:
            check(o, ref, f"flagged outputs, epoch {epoch}")
        assert np.all(done.cpu().numpy() == epoch) and not tiles.cpu().numpy().any(), f"epoch {epoch}"


def test_compute_consumer_ragged_chunks():
    """Two ubatches on two streams, chunks that are not a whole number of
    consumer tiles and a ragged last chunk per ubatch; the consumer (on a
    third stream, queued last) runs FMA work on every word it copies.  Its
    copy of the reduced output must equal the oracle, with no timeouts."""
    P, rows, hidden = 6, 1000, 8192
    n = rows * hidden
    chunk = 1000 * 1024                       # 512000 elements: 62.5 consumer tiles
    ub = [437, 563]
    xs = synth.rank_buffers("normal", P, n, 92)
    ref = oracle.reduce_seq(xs)
    ins = [up16(x) for x in xs]
    outs = [torch.full((n,), 0x5A5A, dtype=torch.int16, device=DEV) for _ in range(P)]
    dst = torch.full((n,), 0x1111, dtype=torch.int16, device=DEV)
    nchunks = tar.ubatch_chunk_count(rows, hidden, 2, ub, chunk)
    done, tiles = u32(nchunks), u32(nchunks)
    timeouts = u32(1)
    grid = 256
    sink = torch.zeros(grid * 256, dtype=torch.float32, device=DEV)
    B = bench_lib()
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    cons = torch.cuda.Stream()
    torch.cuda.synchronize()
    note("compute consumer, ragged chunks")
    tar.ar_reduce_ubatch_flags(ins, outs, rows, hidden, done, tiles, 3, 2, ub, chunk,
                               tar.AR_VARIANT_2STAGE, s)
    # the consumer walks each ubatch's chunks against that ubatch's range
    first, e0 = 0, 0
    for r in ub:
        m = r * hidden
        rc = B.arb_consume_chunks(done.data_ptr(), 3, outs[5].data_ptr() + 2 * e0, dst.data_ptr() + 2 * e0,
                                  m, chunk // 2, first, 1 << 22, timeouts.data_ptr(), 16,
                                  sink.data_ptr(), grid, cons.cuda_stream)
        assert rc == 0
        first += -(-m // (chunk // 2))
        e0 += m
    assert first == nchunks
    torch.cuda.synchronize()
    assert int(timeouts.item()) == 0
    check(dst, ref, "consumer copy")
    assert torch.isfinite(sink).all()


def test_consumer_forced_timeout():
    """Waiting for an epoch that is never published, with a spin limit of 2:
    every tile times out exactly once (here one tile per chunk; one
    wavefront per workgroup polls)."""
    n, chunk_elems = 64 * 8192, 8192
    nchunks = n // chunk_elems
    done = u32(nchunks)
    src = torch.zeros(n, dtype=torch.int16, device=DEV)
    dst = torch.empty(n, dtype=torch.int16, device=DEV)
    timeouts = u32(1)
    note("consumer forced timeout")
    rc = bench_lib().arb_consume_chunks(done.data_ptr(), 9, src.data_ptr(), dst.data_ptr(), n, chunk_elems,
                                        0, 2, timeouts.data_ptr(), 0, None, 16,
                                        torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert int(timeouts.item()) == nchunks
