"""A/B of sequence-number validation on unpack: the library's wavefront
ballot (one compare per word, one ballot per wavefront, two atomics from one
lane of a wavefront that saw a bad word) against per-lane atomics (every
lane with a bad word updates the shared count and minimum itself; the bench
library's arb_unpack_lane_atomics, same loads and stores).  One rank buffer
of bf16 [16384 x 8192] packed with sequence number 5; unpacked expecting 5
(clean: no word bad) and expecting 6 (stale: every word bad).  Prints the
time per variant and checks both report the same count and first index;
run it under rocprofv3 for the per-kernel durations.

Usage:
  python -m tensor_all_reduce_amd.ab_validation [--rounds 5]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--rounds", type=int, default=5)
    a = ap.parse_args(argv)

    import torch

    import tensor_all_reduce_amd as tar
    from tensor_all_reduce_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    tar.lib()
    blib = ctypes.CDLL(os.path.join(os.path.dirname(tar.lib_path), "libarbench.so"))
    vp = ctypes.c_void_p
    blib.arb_unpack_lane_atomics.restype = ctypes.c_int
    blib.arb_unpack_lane_atomics.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_uint32, vp, vp]
    dev = torch.device("cuda:0")
    n = 16384 * 8192
    x = synth.device_rank_buffers("normal", 1, n, 4, dev)[0].view(torch.int16)
    w = torch.empty(n // 2, dtype=torch.int64, device=dev)
    tar.ar_pack_fused(x, w, 5)
    out = torch.empty(n, dtype=torch.int16, device=dev)
    err = torch.empty(2, dtype=torch.int64, device=dev)
    s = torch.cuda.current_stream()

    def lib_unpack(seq):
        tar.ar_err_init(err, stream=s)
        tar.ar_unpack_fused(w, out, seq, err, stream=s)

    def lane_unpack(seq):
        tar.ar_err_init(err, stream=s)
        if blib.arb_unpack_lane_atomics(w.data_ptr(), out.data_ptr(), n, seq, err.data_ptr(), s.cuda_stream) != 0:
            raise RuntimeError("arb_unpack_lane_atomics failed")

    results = {}
    for case, seq in (("clean", 5), ("stale", 6)):
        for name, fn in (("wavefront ballot (library)", lib_unpack), ("per-lane atomics", lane_unpack)):
            ts = []
            for _ in range(a.rounds):
                fn(seq)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                fn(seq)
                e1.record(s)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1))
            got = err.cpu().tolist()
            results[(case, name)] = got
            if not torch.equal(out, x):
                raise SystemExit(f"{name}: unpacked data differs")
            print(f"{case:6s} {name:28s} {statistics.median(ts):9.4f} ms  count {got[0]}  first {got[1]}", flush=True)
        if results[(case, "wavefront ballot (library)")] != results[(case, "per-lane atomics")]:
            raise SystemExit(f"{case}: the two variants report different errors")
    return 0


if __name__ == "__main__":
    sys.exit(main())
