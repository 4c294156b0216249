"""Waiting unpack (ar_unpack_fused_wait): the receiver polls fused payload
words until they carry the expected sequence number, with a bounded spin.

Every case terminates by construction: each wavefront polls at most
max_spins times.  Timeouts are forced from the host (an expected sequence
number that is never written, or words the producer never writes, with a
small spin limit), never by a device-side fault.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_amd as tar
from tensor_all_reduce_amd import synth
from gpu_util import DEV, note, up16, down16, up64, empty16, new_err, err_host

pytestmark = pytest.mark.gpu


def test_wait_payload_already_written():
    n = 3 * 8192 + 6
    x = synth.normal(n, 80)
    w = up64(oracle.pack(x, 41))
    out = empty16(n)
    err = new_err()
    note("unpack_wait ready")
    tar.ar_unpack_fused_wait(w, out, 41, err, max_spins=1000)
    torch.cuda.synchronize()
    want, oe = oracle.unpack(oracle.pack(x, 41), 41)
    assert np.array_equal(down16(out), want)
    assert err_host(err) == (0, 2 ** 64 - 1)


def test_wait_forced_timeout_counts_every_word():
    """Expected sequence number never written, spin limit 3: every word times
    out, is counted exactly once, and its data is still written."""
    n = 64 * 1024 + 2
    x = synth.normal(n, 81)
    w = up64(oracle.pack(x, 7))
    out = empty16(n)
    err = new_err()
    note("unpack_wait forced timeout")
    tar.ar_unpack_fused_wait(w, out, 8, err, max_spins=3)
    torch.cuda.synchronize()
    assert err_host(err) == (n // 2, 0)
    assert np.array_equal(down16(out), x)


def _delay(stream, reps=20):
    """Queue unrelated library work on `stream` so a later launch starts late."""
    P, m = 8, 8 << 20
    ins = [torch.zeros(m, dtype=torch.int16, device=DEV) for _ in range(P)]
    outs = [torch.empty(m, dtype=torch.int16, device=DEV) for _ in range(P)]
    for _ in range(reps):
        tar.ar_reduce_2stage(ins, outs, stream=stream)
    return ins, outs


def test_wait_for_concurrent_producer():
    """The producer packs the data on one stream behind ~2 ms of other work;
    the consumer is queued on another stream right after and polls stale
    payloads (previous sequence number) until the fresh ones land.  It must
    pick up every word with no timeout, and its output equals the oracle's
    unpack.  (If the two streams share a hardware queue the consumer simply
    runs after the producer; the expected result is the same.)"""
    n = 128 * 8192
    x = synth.normal(n, 82)
    ref_words = oracle.pack(x, 100)
    w = up64(oracle.pack(synth.normal(n, 83), 99))     # stale payload from the previous call
    src = up16(x)
    out = empty16(n)
    err = new_err()
    cons, prod = torch.cuda.Stream(), torch.cuda.Stream()
    keep = _delay(prod, reps=1)            # first use of both streams outside the timed part
    tar.ar_err_init(err, stream=cons)
    torch.cuda.synchronize()
    note("unpack_wait concurrent producer")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    keep = _delay(prod)
    tar.ar_pack_fused(src, w, 100, stream=prod)
    e0.record(cons)
    tar.ar_unpack_fused_wait(w, out, 100, err, max_spins=1 << 21, stream=cons)
    e1.record(cons)
    torch.cuda.synchronize()
    print(f"[gpu] waiting unpack ran {e0.elapsed_time(e1):.3f} ms (the producer sat behind ~2 ms of work)")
    want, _ = oracle.unpack(ref_words, 100)
    assert err_host(err) == (0, 2 ** 64 - 1)
    assert np.array_equal(down16(out), want)
    del keep


def test_wait_partial_producer_times_out_exactly():
    """The producer writes only the first half of the payload; the consumer
    reports exactly the words never written, starting at the first of them,
    and the written half matches the oracle."""
    n = 32 * 8192
    W = n // 2
    x = synth.normal(n, 84)
    w = up64(oracle.pack(synth.normal(n, 85), 1))       # stale everywhere
    half = up16(x[: n // 2])
    out = empty16(n)
    err = new_err()
    torch.cuda.synchronize()
    cons, prod = torch.cuda.Stream(), torch.cuda.Stream()
    note("unpack_wait partial producer")
    tar.ar_pack_fused(half, w, 2, n=n // 2, stream=prod)
    tar.ar_unpack_fused_wait(w, out, 2, err, max_spins=200000, stream=cons)
    torch.cuda.synchronize()
    assert err_host(err) == (W - W // 2, W // 2)
    assert np.array_equal(down16(out)[: n // 2], x[: n // 2])


def test_wait_consumes_while_producer_runs(record_property):
    """The pack writes its payload words through to the device-coherent
    level as it stores them (its default SC1 store policy), so a waiting
    unpack running beside it on another stream takes each word as soon as it
    lands rather than when the pack kernel ends.  A 256 MiB payload is
    packed on one stream while the waiting unpack runs on another: the
    consumer finishes well within its own run time after the producer ends
    (it had already taken most of the words; a consumer that could only
    start once the pack ended would need its whole run time after it), and
    its output equals the oracle's unpack.  The lag is measured between an event after the pack
    and an event after the unpack; the consumer's own run time is measured
    on payloads already written."""
    n = 64 << 20                       # 128 MiB of bf16, 256 MiB of payload
    x = synth.normal(n, 86)
    src = up16(x)
    w = torch.empty(n // 2, dtype=torch.int64, device=DEV)
    out = empty16(n)
    err = new_err()
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # warm both streams and time the consumer alone on ready payloads
    tar.ar_pack_fused(src, w, 1, stream=prod)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record(cons)
    tar.ar_unpack_fused_wait(w, out, 1, err, stream=cons)
    b.record(cons)
    torch.cuda.synchronize()
    alone = a.elapsed_time(b)
    lags, packs = [], []
    for k in range(5):
        seq = 10 + k
        tar.ar_err_init(err, stream=cons)
        torch.cuda.synchronize()
        p0, p1, c1 = ev(), ev(), ev()
        note(f"unpack_wait beside a running pack, seq {seq}")
        p0.record(prod)
        tar.ar_pack_fused(src, w, seq, stream=prod)
        p1.record(prod)
        tar.ar_unpack_fused_wait(w, out, seq, err, max_spins=1 << 22, stream=cons)
        c1.record(cons)
        torch.cuda.synchronize()
        assert err_host(err) == (0, 2 ** 64 - 1)
        packs.append(p0.elapsed_time(p1))
        lags.append(p1.elapsed_time(c1))
    want, _ = oracle.unpack(oracle.pack(x, 14), 14)
    assert np.array_equal(down16(out), want)
    lag = min(lags)
    print(f"[gpu] pack {min(packs):.3f} ms; waiting unpack alone {alone:.3f} ms; consumer end after producer end "
          f"{', '.join(f'{v:.3f}' for v in lags)} ms")
    record_property("consumer_alone_ms", round(alone, 4))
    record_property("consumer_lag_after_producer_ms", [round(v, 4) for v in lags])
    assert lag < 0.7 * alone
