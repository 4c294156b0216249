"""A/B of the access width for the fused 8 -> 8 reduce: 4-, 8- and 16-byte
accesses per lane (global_load_dword / _dwordx2 / _dwordx4 and the matching
stores), with the same tiles (64-lane workgroups owning 1 KiB of every
buffer), the same bytes in flight per lane, the same arithmetic and the same
occupancy caps; the bench library's arb_width_reduce8.  The library's own
fused two-stage (16-byte accesses) runs beside them at its default shape.
P = 8 buffers of bf16 [16384 x 8192].  Prints GB/s per variant (medians of
interleaved rounds) and checks that every variant produced the library's
result; run it under rocprofv3 for per-kernel durations and counters
(SQ_INSTS_VMEM_RD / _WR show the instruction count scale with 16 / width).

Usage:
  python -m tensor_all_reduce_amd.ab_loadwidth [--rounds 5]
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
    blib.arb_width_reduce8.restype = ctypes.c_int
    blib.arb_width_reduce8.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_int, vp]
    dev = torch.device("cuda:0")
    P, n = 8, 16384 * 8192
    ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, n, 4, dev)]
    outs = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(P)]
    ref = torch.empty(n, dtype=torch.int16, device=dev)
    tar.ar_reduce_oneshot(ins, ref)
    s = torch.cuda.current_stream()
    ip = (vp * P)(*[x.data_ptr() for x in ins])
    op = (vp * P)(*[o.data_ptr() for o in outs])

    def lib():
        tar.ar_reduce_2stage(ins, outs)

    def width(w, wg):
        def f():
            if blib.arb_width_reduce8(ip, op, n, w, wg, s.cuda_stream) != 0:
                raise RuntimeError("arb_width_reduce8 failed")
        return f

    shape = tar.ar_get_launch_shape(tar.AR_KERNEL_2STAGE)
    variants = {f"library two-stage, 16-byte accesses, shape {tuple(shape)}": lib}
    for wg in (4, 6, 8):
        for w in (16, 8, 4):
            variants[f"{w:2d}-byte accesses, 64-lane workgroups, {wg} per CU"] = width(w, wg)
    times = {k: [] for k in variants}
    for _ in range(a.rounds):
        for name, fn in variants.items():
            fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(3):
                fn()
            e1.record(s)
            e1.synchronize()
            times[name].append(e0.elapsed_time(e1) / 3)
            for o in (outs[0], outs[-1]):
                if not torch.equal(o, ref):
                    raise SystemExit(f"{name}: result differs from the library's")
    credited = 2 * P * 2 * n
    for name, t in times.items():
        ms = statistics.median(t)
        print(f"{name:60s} {ms:8.4f} ms  {credited / (ms * 1e-3) / 1e9:8.1f} GB/s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
