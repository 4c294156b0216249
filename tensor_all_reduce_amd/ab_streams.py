"""Attainable bandwidth against the number of concurrent streams: N buffers
copied side by side into N others (out[j] = in[j], no arithmetic; the bench
library's arb_copy_multi) for N = 1, 2, 4 and 8, 4 GiB moved per call
whatever N, uncapped and at several workgroups-per-CU caps.  The 8 -> 8 case
is the access pattern of the fused two-stage and recursive-doubling kernels;
the 1 -> 1 case is a plain copy.  Then the one-shot's 8 -> 1 pattern: eight
256 MiB buffers gathered into one by XOR (the bench library's
arb_gather_xor: the one-shot's tiling, no float work) over store kind and
cap, with the library's one-shot on the same buffers beside it.  Prints GB/s
per case (medians of interleaved rounds).

Usage:
  python -m tensor_all_reduce_amd.ab_streams [--rounds 3]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--rounds", type=int, default=3)
    a = ap.parse_args(argv)

    import torch

    import tensor_all_reduce_amd as tar

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    tar.lib()
    blib = ctypes.CDLL(os.path.join(os.path.dirname(tar.lib_path), "libarbench.so"))
    vp = ctypes.c_void_p
    blib.arb_copy_multi.restype = ctypes.c_int
    blib.arb_copy_multi.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_int, vp]
    blib.arb_gather_xor.restype = ctypes.c_int
    blib.arb_gather_xor.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                    vp]
    dev = torch.device("cuda:0")
    total = 4 << 30                                  # bytes moved per call (read + write)
    s = torch.cuda.current_stream()
    bufs = {}
    for nb in (1, 2, 4, 8):
        per = total // 2 // nb                       # bytes per buffer
        ins = [torch.empty(per, dtype=torch.uint8, device=dev) for _ in range(nb)]
        outs = [torch.empty(per, dtype=torch.uint8, device=dev) for _ in range(nb)]
        for t in ins:
            t.fill_(1)
        bufs[nb] = (ins, outs, per, (vp * nb)(*[t.data_ptr() for t in ins]), (vp * nb)(*[t.data_ptr() for t in outs]))
    cases = [(nb, vec, wg) for nb in (1, 2, 4, 8) for vec in (1, 2) for wg in (0, 4, 5, 6, 8)]
    res = {c: [] for c in cases}
    for _ in range(a.rounds):
        for c in cases:
            nb, vec, wg = c
            _, _, per, ip, op = bufs[nb]

            def f():
                if blib.arb_copy_multi(ip, op, nb, per, vec, wg, s.cuda_stream) != 0:
                    raise RuntimeError("arb_copy_multi failed")
            f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(5):
                f()
            e1.record(s)
            e1.synchronize()
            res[c].append(total / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9)
    for nb in (1, 2, 4, 8):
        best = max(cases, key=lambda c: statistics.median(res[c]) if c[0] == nb else -1)
        unc = statistics.median(res[(nb, 1, 0)])
        print(f"{nb} -> {nb}: uncapped (1 group per lane) {unc:7.1f} GB/s; best {statistics.median(res[best]):7.1f} GB/s "
              f"at {best[1]} group(s) per lane, {best[2] or 'no'} cap", flush=True)
    print("all cases (GB/s, median):")
    for c in cases:
        print(f"  {c[0]} -> {c[0]}  vec {c[1]}  wg/cu {c[2]:2d}  {statistics.median(res[c]):7.1f}")
    del bufs
    torch.cuda.empty_cache()
    # 8 -> 1: the one-shot's pattern, P = 8 buffers of bf16 [16384 x 8192]
    P, n = 8, 16384 * 8192
    ins = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(P)]
    for j, t in enumerate(ins):
        t.fill_(j + 1)
    out = torch.empty(n, dtype=torch.int16, device=dev)
    ip = (vp * P)(*[t.data_ptr() for t in ins])
    moved = (P + 1) * 2 * n
    gcases = [("gather", nts, wg) for nts in (0, 1) for wg in (0, 4, 8, 12, 16)] + [("one-shot", None, None)]
    gres = {c: [] for c in gcases}
    for _ in range(a.rounds):
        for c in gcases:
            if c[0] == "gather":
                def f(c=c):
                    if blib.arb_gather_xor(ip, P, out.data_ptr(), 2 * n, c[1], c[2], s.cuda_stream) != 0:
                        raise RuntimeError("arb_gather_xor failed")
            else:
                def f():
                    tar.ar_reduce_oneshot(ins, out)
            f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(5):
                f()
            e1.record(s)
            e1.synchronize()
            gres[c].append(moved / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9)
    print(f"8 -> 1 (GB/s, median; one-shot shape {tuple(tar.ar_get_launch_shape(tar.AR_KERNEL_ONESHOT))}):")
    for c in gcases:
        name = "library one-shot" if c[0] == "one-shot" else f"gather  nt_stores {c[1]}  wg/cu {c[2]:2d}"
        print(f"  {name:34s} {statistics.median(gres[c]):7.1f}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
