"""Profiling target for the kernels beyond the bench step: the fp8 path
(quantise all 8 ranks, reduce into one output and into all 8), the flagged
two-stage ubatch reduce (per-chunk completion flags, both ubatches on one
stream), the same ubatch reduce on its bounded-footprint grid, and the
waiting unpack on payloads that already carry the expected sequence number,
each `reps` times at the prefill shape (P = 8, bf16 [16384 x 8192] per
rank), then three plain copies of exactly 1 GiB that calibrate FETCH_SIZE /
WRITE_SIZE.  No call here waits on another stream, so
it can run under counter collection, which serialises kernels.

Usage: python -m tensor_all_reduce_amd.frows_trace [--reps 4]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--reps", type=int, default=4)
    a = ap.parse_args(argv)

    import torch

    import tensor_all_reduce_amd as tar
    from tensor_all_reduce_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    tar.lib()
    blib = ctypes.CDLL(os.path.join(os.path.dirname(tar.lib_path), "libarbench.so"))
    vp = ctypes.c_void_p
    blib.arb_copy.restype = ctypes.c_int
    blib.arb_copy.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
    dev = torch.device("cuda:0")
    P, rows, hidden = 8, 16384, 8192
    n = rows * hidden
    ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, n, 4, dev)]
    outs = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(P)]
    codes = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(P)]
    scales = [torch.empty(tar.fp8_scale_count(n), dtype=torch.uint8, device=dev) for _ in range(P)]
    for _ in range(a.reps):
        tar.ar_quantize_fp8(ins, codes, scales)
    for _ in range(a.reps):
        tar.ar_reduce_fp8(codes, scales, outs[:1])
    for _ in range(a.reps):
        tar.ar_reduce_fp8(codes, scales, outs)
    torch.cuda.synchronize()
    print("[frows] fp8 done", flush=True)
    del codes, scales
    nflags = tar.ubatch_chunk_count(rows, hidden, 2, None, 1 << 20)
    done = torch.zeros(nflags, dtype=torch.int32, device=dev)
    tiles = torch.zeros(nflags, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    for r in range(a.reps):
        tar.ar_reduce_ubatch_flags(ins, outs, rows, hidden, done, tiles, r + 1, 2, None, 1 << 20,
                                   tar.AR_VARIANT_2STAGE, [s, s])
    torch.cuda.synchronize()
    if not bool((done == a.reps).all()) or bool(tiles.any()):
        raise SystemExit("flagged reduce: flags or counters not as expected")
    print("[frows] flagged ubatch done", flush=True)
    for _ in range(a.reps):
        tar.ar_reduce_ubatch(ins, outs, rows, hidden, 2, None, 1 << 20,
                             tar.AR_VARIANT_2STAGE | tar.AR_UBATCH_BOUNDED, [s, s])
    torch.cuda.synchronize()
    print("[frows] bounded ubatch done", flush=True)
    del outs
    torch.cuda.empty_cache()
    words = [torch.empty(n // 2, dtype=torch.int64, device=dev) for _ in range(P)]
    for p in range(P):
        tar.ar_pack_fused(ins[p], words[p], 7)
    err = torch.empty(2, dtype=torch.int64, device=dev)
    tar.ar_err_init(err)
    xo = torch.empty(n, dtype=torch.int16, device=dev)
    for _ in range(a.reps):
        for p in range(P):
            tar.ar_unpack_fused_wait(words[p], xo, 7, err)
    torch.cuda.synchronize()
    if int(err[0].item()) != 0:
        raise SystemExit("waiting unpack counted stale words")
    print("[frows] waiting unpack done", flush=True)
    del words, ins
    torch.cuda.empty_cache()
    cb = 1 << 30
    src = torch.empty(cb // 2, dtype=torch.int16, device=dev)
    dst = torch.empty(cb // 2, dtype=torch.int16, device=dev)
    src.fill_(1)
    for _ in range(3):
        if blib.arb_copy(src.data_ptr(), dst.data_ptr(), cb, 64, s.cuda_stream) != 0:
            raise SystemExit("arb_copy failed")
    torch.cuda.synchronize()
    print("[frows] calibration copies done", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
