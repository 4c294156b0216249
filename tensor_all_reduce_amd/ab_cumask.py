"""The ubatch reduce beside a GEMM, with the GPU's compute units split
between them by CU-masked streams.

One ubatch of the two-stage reduce (P = 8 buffers of bf16 [8192 x 8192],
1 MiB chunks) runs on one stream and three bf16 GEMMs [4096 x 4096] x
[4096 x 4096] (torch.mm, the partner ubatch's compute) on another: alone,
then both at once.  overlap = (t_reduce + t_gemm - t_both) / min(t_reduce,
t_gemm).  Cases: plain streams; both streams masked to every CU (the cost of
a mask by itself); and the reduce on the first k CUs of the mask with the
GEMM on the rest.  Masks set contiguous bits, which spread over all eight
XCDs.  Every reduce output is checked against the one-shot result.

The masked streams are made by hipExtStreamCreateWithCUMask in the HIP
runtime the process already loaded (torch's); a CU mask needs its own
hardware queue, so each case runs in a process of its own, started from
this one, which itself never touches the GPU.

Usage: python -m tensor_all_reduce_amd.ab_cumask [--splits 32,64,96,128,192]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys


def one(cfg: str) -> int:
    import ctypes

    import torch

    import tensor_all_reduce_amd as tar
    from tensor_all_reduce_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    tar.lib()
    dev = torch.device("cuda:0")
    torch.zeros(1, device=dev)
    path = [ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln][0]
    hip = ctypes.CDLL(path)
    hip.hipExtStreamCreateWithCUMask.restype = ctypes.c_int
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    P, rows, H = 8, 8192, 8192
    m = rows * H
    ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, m, 4, dev)]
    outs = [torch.empty(m, dtype=torch.int16, device=dev) for _ in range(P)]
    ref = torch.empty(m, dtype=torch.int16, device=dev)
    tar.ar_reduce_oneshot(ins, ref)
    ga = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    gb = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    gc = torch.empty(4096, 4096, device=dev, dtype=torch.bfloat16)
    main = torch.cuda.current_stream()

    def masked(bits):
        nw = (cus + 31) // 32
        words = (ctypes.c_uint32 * nw)()
        for b in bits:
            words[b // 32] |= 1 << (b % 32)
        h = ctypes.c_void_p()
        rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), nw, words)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask returned {rc}")
        return torch.cuda.ExternalStream(h.value)

    if cfg == "plain":
        label, sa, sg = "plain streams", torch.cuda.Stream(), torch.cuda.Stream()
    elif cfg == "full":
        label, sa, sg = "both masked to all CUs", masked(range(cus)), masked(range(cus))
    else:
        k = int(cfg)
        label = f"reduce on {k} CUs, GEMM on {cus - k}"
        sa, sg = masked(range(k)), masked(range(k, cus))

    def red():
        sa.wait_stream(main)
        tar.ar_reduce_ubatch(ins, outs, rows, H, 1, None, 1 << 20, tar.AR_VARIANT_2STAGE, streams=[sa])
        main.wait_stream(sa)

    def gem():
        sg.wait_stream(main)
        with torch.cuda.stream(sg):
            for _ in range(3):
                torch.mm(ga, gb, out=gc)
        main.wait_stream(sg)

    def both():
        sa.wait_stream(main)
        sg.wait_stream(main)
        tar.ar_reduce_ubatch(ins, outs, rows, H, 1, None, 1 << 20, tar.AR_VARIANT_2STAGE, streams=[sa])
        with torch.cuda.stream(sg):
            for _ in range(3):
                torch.mm(ga, gb, out=gc)
        main.wait_stream(sa)
        main.wait_stream(sg)

    def timed(fn, reps=10):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(main)
            fn()
            e1.record(main)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    tr, tg, tb = timed(red), timed(gem), timed(both)
    if not all(torch.equal(o, ref) for o in outs):
        raise SystemExit(f"{label}: reduce output differs from the one-shot result")
    print(json.dumps({"case": label, "reduce_ms": round(tr, 4), "gemm_ms": round(tg, 4), "both_ms": round(tb, 4),
                      "serial_ms": round(tr + tg, 4), "overlap": round((tr + tg - tb) / min(tr, tg), 3)}),
          flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--splits", default="32,64,96,128,192", help="CUs given to the reduce")
    ap.add_argument("--one", default=None, help=argparse.SUPPRESS)
    a = ap.parse_args(argv)
    if a.one is not None:
        return one(a.one)
    cases = ["plain", "full"] + [s for s in a.splits.split(",") if s]
    print("case                                reduce ms   GEMM ms   both ms  serial ms  overlap", flush=True)
    for c in cases:
        r = subprocess.run([sys.executable, "-m", "tensor_all_reduce_amd.ab_cumask", "--one", c],
                           capture_output=True, text=True, timeout=300,
                           cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        line = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not line:
            print(f"{c}: failed (exit {r.returncode}): {(r.stderr or r.stdout).strip().splitlines()[-1:]}",
                  flush=True)
            return 1
        d = json.loads(line[-1])
        print(f"{d['case']:34s} {d['reduce_ms']:9.3f} {d['gemm_ms']:9.3f} {d['both_ms']:9.3f} "
              f"{d['serial_ms']:10.3f} {d['overlap']:8.2f}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
