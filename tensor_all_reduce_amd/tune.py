"""Launch-shape tuner: measures every candidate shape of each kernel kind on
one GPU, in one process, and prints the ranking.

Workload: P = 8 bf16 buffers of [16384 x 8192] (256 MiB each), N(0,1), the
same batch bench.py times.  Pack and unpack run once per rank buffer (8
calls over 8 different buffers), as in the bench step, so no buffer is
re-read from the 256 MiB last-level cache.  For each kind, every candidate (block, vec,
nt_loads, nt_stores, wg_per_cu) is set with ar_set_launch_shape and timed
with HIP events around `reps` back-to-back calls; candidates are visited in a
shuffled order each round and the median over rounds is reported, so slow
drift of the device affects all candidates alike.  GB/s counts each input
read once and each output written once.

With --decode, the one-shot and fused two-stage kernels are instead timed at
the decode sizes (P = 8, [T x 8192] for T = 8, 32, 128: 128 KiB to 2 MiB per
buffer) as per-call stream time over 2000 back-to-back calls from the native
timing loop in libarbench.so, so no Python runs between calls.

Usage: python -m tensor_all_reduce_amd.tune [--kinds 2stage,rd] [--rounds 3] [--reps 4]
       python -m tensor_all_reduce_amd.tune --decode
"""
from __future__ import annotations

import argparse
import itertools
import random
import statistics
import sys

import torch

import tensor_all_reduce_amd as tar
from tensor_all_reduce_amd import synth

P, ROWS, HIDDEN = 8, 16384, 8192
WGS = (0, 2, 3, 4, 5, 6, 8, 10, 12, 16)
KINDS = {
    "oneshot": tar.AR_KERNEL_ONESHOT, "2stage": tar.AR_KERNEL_2STAGE, "ubatch": tar.AR_KERNEL_UBATCH,
    "rs": tar.AR_KERNEL_RS, "ag": tar.AR_KERNEL_AG, "pack": tar.AR_KERNEL_PACK,
    "unpack": tar.AR_KERNEL_UNPACK, "rd": tar.AR_KERNEL_RD, "rdstep": tar.AR_KERNEL_RDSTEP,
    "ubatch_flags": tar.AR_KERNEL_UBATCH_FLAGS, "quant_fp8": tar.AR_KERNEL_QUANT_FP8,
    "reduce_fp8": tar.AR_KERNEL_REDUCE_FP8_ALL, "reduce_fp8_one": tar.AR_KERNEL_REDUCE_FP8,
}


def candidates(kind: str):
    vecs = (1, 2) if kind in ("oneshot", "2stage", "ubatch", "ubatch_flags", "quant_fp8", "reduce_fp8",
                              "reduce_fp8_one", "rd", "pack", "unpack") else (1,)
    return list(itertools.product((64, 128, 256), vecs, (0, 1), (0, 1), WGS))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--kinds", default="oneshot,2stage,ubatch,pack,unpack,rd")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--reps", type=int, default=4)
    ap.add_argument("--top", type=int, default=8)
    ap.add_argument("--decode", action="store_true", help="tune the decode-size latency instead")
    args = ap.parse_args(argv)
    if args.decode:
        return decode(args)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = ROWS * HIDDEN
    W = n // 2
    ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, n, 4, dev)]
    outs = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(P)]
    scratch = torch.empty(n, dtype=torch.int16, device=dev)
    words = [torch.empty(W, dtype=torch.int64, device=dev) for _ in range(P)]
    rdo = [torch.empty(W, dtype=torch.int64, device=dev) for _ in range(P)]
    mailbox = torch.empty(tar.rd_mailbox_words(P, n), dtype=torch.int64, device=dev)
    err = torch.empty(2, dtype=torch.int64, device=dev)
    main_s = torch.cuda.current_stream()
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    B = 2 * n
    nflags = tar.ubatch_chunk_count(ROWS, HIDDEN, 2, None, 1 << 20)
    done = torch.zeros(nflags, dtype=torch.int32, device=dev)
    tiles = torch.zeros(nflags, dtype=torch.int32, device=dev)
    epoch = [0]
    for r in range(P):
        tar.ar_pack_fused(ins[r], words[r], 1)
    tar.ar_err_init(err)
    codes = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(P)]
    scales = [torch.empty(tar.fp8_scale_count(n), dtype=torch.uint8, device=dev) for _ in range(P)]
    tar.ar_quantize_fp8(ins, codes, scales)

    def op(kind):
        if kind == "oneshot":
            tar.ar_reduce_oneshot(ins, outs[0])
        elif kind == "2stage":
            tar.ar_reduce_2stage(ins, outs)
        elif kind in ("rs", "ag"):
            tar.ar_reduce_2stage(ins, outs, scratch=scratch)
        elif kind == "ubatch":
            s0.wait_stream(main_s)
            s1.wait_stream(main_s)
            tar.ar_reduce_ubatch(ins, outs, ROWS, HIDDEN, 2, None, 1 << 20, tar.AR_VARIANT_2STAGE, [s0, s1])
            main_s.wait_stream(s0)
            main_s.wait_stream(s1)
        elif kind == "ubatch_flags":
            epoch[0] += 1
            s0.wait_stream(main_s)
            s1.wait_stream(main_s)
            tar.ar_reduce_ubatch_flags(ins, outs, ROWS, HIDDEN, done, tiles, epoch[0], 2, None, 1 << 20,
                                       tar.AR_VARIANT_2STAGE, [s0, s1])
            main_s.wait_stream(s0)
            main_s.wait_stream(s1)
        elif kind == "pack":
            for r in range(P):
                tar.ar_pack_fused(ins[r], words[r], 1)
        elif kind == "unpack":
            for r in range(P):
                tar.ar_unpack_fused(words[r], outs[r], 1, err)
        elif kind == "rd":
            tar.ar_rd_schedule(words, rdo, 1, err)
        elif kind == "rdstep":
            tar.ar_rd_schedule(words, rdo, 1, err, mailbox=mailbox, flags=tar.AR_RD_STAGED)
        elif kind == "quant_fp8":
            tar.ar_quantize_fp8(ins, codes, scales)
        elif kind == "reduce_fp8":
            tar.ar_reduce_fp8(codes, scales, outs)
        elif kind == "reduce_fp8_one":
            tar.ar_reduce_fp8(codes, scales, outs[:1])

    credited = {"oneshot": (P + 1) * B, "2stage": 2 * P * B, "ubatch": 2 * P * B, "ubatch_flags": 2 * P * B,
                "rs": 2 * P * B,
                "ag": 2 * P * B, "pack": 3 * P * B, "unpack": 3 * P * B, "rd": 4 * P * B, "rdstep": 4 * P * B,
                "quant_fp8": P * (3 * n + tar.fp8_scale_count(n)),
                "reduce_fp8": P * (n + tar.fp8_scale_count(n)) + P * B,
                "reduce_fp8_one": P * (n + tar.fp8_scale_count(n)) + B}

    def time_one(kind):
        op(kind)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main_s)
        for _ in range(args.reps):
            op(kind)
        e1.record(main_s)
        e1.synchronize()
        return e0.elapsed_time(e1) / args.reps

    rng = random.Random(7)
    for kind in args.kinds.split(","):
        k = KINDS[kind]
        default = tar.ar_get_launch_shape(k)
        cands = candidates(kind)
        if default not in cands:
            cands.append(default)
        times = {c: [] for c in cands}
        for rnd in range(args.rounds):
            order = cands[:]
            rng.shuffle(order)
            for c in order:
                tar.ar_set_launch_shape(k, *c)
                times[c].append(time_one(kind))
            print(f"[tune] {kind}: round {rnd + 1}/{args.rounds} done", file=sys.stderr, flush=True)
        tar.ar_set_launch_shape(k, *default)
        med = {c: statistics.median(v) for c, v in times.items()}
        ranked = sorted(cands, key=lambda c: med[c])
        print(f"== {kind}: credited {credited[kind]} B per call, {len(cands)} shapes, "
              f"{args.rounds} rounds x {args.reps} calls")
        print("   rank  block vec ntl nts wg/cu      ms      GB/s  frac-of-8TB/s")
        for i, c in enumerate(ranked):
            if i < args.top or c == default:
                gbps = credited[kind] / (med[c] * 1e-3) / 1e9
                tag = "  <- default" if c == default else ""
                print(f"   {i + 1:4d}  {c[0]:5d} {c[1]:3d} {c[2]:3d} {c[3]:3d} {c[4]:5d} {med[c]:8.4f} "
                      f"{gbps:8.1f}  {gbps / 8000:.4f}{tag}")
        sys.stdout.flush()
    torch.cuda.synchronize()
    return 0


def decode(args):
    import ctypes
    import os
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    blib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "libarbench.so"))
    vp = ctypes.c_void_p
    blib.arb_stream_us.restype = ctypes.c_double
    blib.arb_stream_us.argtypes = [ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int,
                                   ctypes.c_size_t, vp, ctypes.c_int, vp]
    sh = torch.cuda.current_stream().cuda_stream
    rng = random.Random(11)
    for T in (8, 32, 128):
        m = T * HIDDEN
        ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, m, 2, dev)]
        outs = [torch.empty(m, dtype=torch.int16, device=dev) for _ in range(P)]
        ia = (vp * P)(*[t.data_ptr() for t in ins])
        oa = (vp * P)(*[t.data_ptr() for t in outs])
        for name, which, k in (("oneshot", 0, tar.AR_KERNEL_ONESHOT), ("2stage", 1, tar.AR_KERNEL_2STAGE)):
            default = tar.ar_get_launch_shape(k)
            cands = list(itertools.product((64, 128, 256), (1, 2), (0, 1), (0, 1), (0,)))
            if default not in cands:
                cands.append(default)
            times = {c: [] for c in cands}
            for _ in range(args.rounds):
                order = cands[:]
                rng.shuffle(order)
                for c in order:
                    tar.ar_set_launch_shape(k, *c)
                    us = blib.arb_stream_us(which, ia, oa, P, m, None, 2000, sh)
                    if us < 0:
                        raise RuntimeError(f"arb_stream_us failed: {us}")
                    times[c].append(us)
            tar.ar_set_launch_shape(k, *default)
            med = {c: statistics.median(v) for c, v in times.items()}
            ranked = sorted(cands, key=lambda c: med[c])
            print(f"== {name} T={T} ({2 * m // 1024} KiB per buffer): per-call stream time")
            print("   rank  block vec ntl nts wg/cu      us")
            for i, c in enumerate(ranked):
                if i < args.top or c == default:
                    tag = "  <- default" if c == default else ""
                    print(f"   {i + 1:4d}  {c[0]:5d} {c[1]:3d} {c[2]:3d} {c[3]:3d} {c[4]:5d} {med[c]:7.2f}{tag}")
            sys.stdout.flush()
    return 0


if __name__ == "__main__":
    sys.exit(main())
