"""A/B of the launch structure for the fused 8 -> 8 reduce: the library's
flat in-order tiles (ar_reduce_2stage) against a grid-stride loop whose grid
is sized to the CU count (1, 2, 4 and 8 workgroups of 256 lanes per CU; the
bench library's arb_gridstride_reduce8, same arithmetic).  P = 8 buffers of
bf16 [16384 x 8192].  Prints GB/s per variant (medians of interleaved rounds)
and checks that every variant produced the library's result; run it under
rocprofv3 to get the per-kernel durations and counters.

Usage:
  python -m tensor_all_reduce_amd.ab_gridstride [--rounds 5]
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
    blib.arb_gridstride_reduce8.restype = ctypes.c_int
    blib.arb_gridstride_reduce8.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_size_t, ctypes.c_int,
                                            vp]
    dev = torch.device("cuda:0")
    P, n = 8, 16384 * 8192
    ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, n, 4, dev)]
    outs = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(P)]
    ref = torch.empty(n, dtype=torch.int16, device=dev)
    tar.ar_reduce_oneshot(ins, ref)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    s = torch.cuda.current_stream()
    ip = (vp * P)(*[x.data_ptr() for x in ins])
    op = (vp * P)(*[o.data_ptr() for o in outs])

    def flat():
        tar.ar_reduce_2stage(ins, outs)

    def gs(mult):
        def f():
            if blib.arb_gridstride_reduce8(ip, op, n, cus * mult, s.cuda_stream) != 0:
                raise RuntimeError("arb_gridstride_reduce8 failed")
        return f

    variants = {"flat in-order tiles (library)": flat}
    for m in (1, 2, 4, 8):
        variants[f"grid-stride, {m} x 256-lane workgroups per CU"] = gs(m)
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
        print(f"{name:48s} {ms:8.4f} ms  {credited / (ms * 1e-3) / 1e9:8.1f} GB/s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
