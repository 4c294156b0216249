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

With --decode, the small-message kinds (one-shot, fused two-stage, fused
recursive doubling, the staged recursive-doubling step, pack and unpack, for
n <= AR_SMALL_ELEMS) are instead timed at the decode sizes (P = 8, [T x 8192]
for T = 8, 32, 128: 128 KiB to 2 MiB per buffer) as per-call time inside a
HIP graph (50 calls captured, replayed): at these sizes back-to-back eager
calls are bound by the host's launch cost, which would hide the kernels'
differences.

With --crossover, the current large-message and small-message default shapes
of those three kernels are both timed at sizes from 128 KiB to 64 MiB per
buffer, hot (one buffer set, repeated) and cold (rotating over >= 4 GiB; the
one-shot and two-stage only), the evidence for the AR_SMALL_ELEMS threshold.

Usage: python -m tensor_all_reduce_amd.tune [--kinds 2stage,rd] [--rounds 3] [--reps 4]
       python -m tensor_all_reduce_amd.tune --decode [--kinds pack,unpack]
       python -m tensor_all_reduce_amd.tune --crossover
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
# The prefill sweep times the large-message kinds: at [16384 x 8192] per rank
# the one-shot, two-stage and RD calls use them, not the ..._SMALL kinds.


def candidates(kind: str):
    vecs = (1, 2) if kind in ("oneshot", "2stage", "ubatch", "ubatch_flags", "quant_fp8", "reduce_fp8",
                              "reduce_fp8_one", "rd", "pack", "unpack") else (1,)
    return list(itertools.product((64, 128, 256), vecs, (0, 1), (0, 1), WGS))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--kinds", default=None,
                    help="kinds to sweep (default oneshot,2stage,ubatch,pack,unpack,rd; with --decode, "
                         "any of oneshot,2stage,rd,rdstep,pack,unpack, default all)")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--reps", type=int, default=4)
    ap.add_argument("--top", type=int, default=8)
    ap.add_argument("--decode", action="store_true", help="tune the decode-size latency instead")
    ap.add_argument("--crossover", action="store_true",
                    help="time the large- and small-message default shapes across sizes")
    args = ap.parse_args(argv)
    args.kinds_given = args.kinds is not None
    if args.kinds is None:
        args.kinds = "oneshot,2stage,ubatch,pack,unpack,rd"
    if args.decode:
        return decode(args)
    if args.crossover:
        return crossover(args)

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


def _bench_lib():
    import ctypes
    import os
    blib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "libarbench.so"))
    vp = ctypes.c_void_p
    pp = ctypes.POINTER(vp)
    blib.arb_stream_us.restype = ctypes.c_double
    blib.arb_stream_us.argtypes = [ctypes.c_int, pp, pp, ctypes.c_int, ctypes.c_size_t, vp, ctypes.c_int, vp]
    blib.arb_stream_rot_us.restype = ctypes.c_double
    blib.arb_stream_rot_us.argtypes = [ctypes.c_int, pp, pp, ctypes.c_int, ctypes.c_size_t, ctypes.c_size_t,
                                       ctypes.c_int, ctypes.c_int, vp]
    blib.arb_decode_us.restype = ctypes.c_double
    blib.arb_decode_us.argtypes = [pp, pp, pp, pp, ctypes.c_int, ctypes.c_size_t, vp, ctypes.c_int, vp,
                                   ctypes.c_int, ctypes.c_int, vp]
    return blib, vp


def _check_us(us, what):
    if us < 0:
        raise RuntimeError(f"{what} failed: {us}")
    return us


def _graph_us(body, per_graph: int = 50, replays: int = 8) -> float:
    """Per-call GPU time of body(stream): `per_graph` calls captured in one
    HIP graph, replayed `replays` times (after one untimed replay)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        body(side)
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            for _ in range(per_graph):
                body(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * per_graph)


def decode(args):
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rng = random.Random(11)
    mmax = 128 * HIDDEN
    ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, mmax, 2, dev)]
    mbox = torch.empty(tar.rd_mailbox_words(P, mmax), dtype=torch.int64, device=dev)
    outs = [torch.empty(mmax, dtype=torch.int16, device=dev) for _ in range(P)]
    words = [torch.empty(mmax // 2, dtype=torch.int64, device=dev) for _ in range(P)]
    rdo = [torch.empty(mmax // 2, dtype=torch.int64, device=dev) for _ in range(P)]
    err = torch.empty(2, dtype=torch.int64, device=dev)
    tar.ar_err_init(err)
    cands = list(itertools.product((64, 128, 256), (1, 2), (0, 1), (0, 1), (0, 4, 8)))
    only = set(args.kinds.split(",")) if args.kinds_given else None
    totals = {}          # name -> {shape: summed per-call us over the decode sizes}
    for T in (8, 32, 128):
        m = T * HIDDEN
        xi, xo = [x[:m] for x in ins], [o[:m] for o in outs]
        wi, wo = [w[:m // 2] for w in words], [w[:m // 2] for w in rdo]
        for p in range(P):
            tar.ar_pack_fused(xi[p], wi[p], 1)

        def pack_all(st):
            for p in range(P):
                tar.ar_pack_fused(xi[p], wi[p], 1, stream=st)

        def unpack_all(st):
            for p in range(P):
                tar.ar_unpack_fused(wi[p], xo[p], 1, err, stream=st)
        # (name, kind, body, calls per body)
        for name, k, body, per in (
                ("oneshot", tar.AR_KERNEL_ONESHOT_SMALL, lambda st: tar.ar_reduce_oneshot(xi, xo[0], stream=st), 1),
                ("2stage", tar.AR_KERNEL_2STAGE_SMALL, lambda st: tar.ar_reduce_2stage(xi, xo, stream=st), 1),
                ("rd", tar.AR_KERNEL_RD_SMALL, lambda st: tar.ar_rd_schedule(wi, wo, 1, err, stream=st), 1),
                ("rdstep", tar.AR_KERNEL_RDSTEP_SMALL,
                 lambda st: tar.ar_rd_schedule(wi, wo, 1, err, mailbox=mbox, flags=tar.AR_RD_STAGED, stream=st), 1),
                ("pack", tar.AR_KERNEL_PACK_SMALL, pack_all, P),
                ("unpack", tar.AR_KERNEL_UNPACK_SMALL, unpack_all, P)):
            if only is not None and name not in only:
                continue
            default = tar.ar_get_launch_shape(k)
            cs = cands + ([default] if default not in cands else [])
            times = {c: [] for c in cs}
            for _ in range(args.rounds):
                order = cs[:]
                rng.shuffle(order)
                for c in order:
                    tar.ar_set_launch_shape(k, *c)
                    try:
                        times[c].append(_graph_us(body, per_graph=max(1, 50 // per)) / per)
                    finally:
                        tar.ar_set_launch_shape(k, *default)
            med = {c: statistics.median(v) for c, v in times.items()}
            tot = totals.setdefault(name, {"default": default})
            for c, v in med.items():
                tot[c] = tot.get(c, 0.0) + v
            ranked = sorted(cs, key=lambda c: med[c])
            what = (f"{4 * m // 1024} KiB of payload per rank" if name.startswith("rd")
                    else f"{2 * m // 1024} KiB per buffer")
            print(f"== {name} (small-message kind) T={T} ({what}): per-call time in a HIP graph")
            print("   rank  block vec ntl nts wg/cu      us")
            for i, c in enumerate(ranked):
                if i < args.top or c == default:
                    tag = "  <- default" if c == default else ""
                    print(f"   {i + 1:4d}  {c[0]:5d} {c[1]:3d} {c[2]:3d} {c[3]:3d} {c[4]:5d} {med[c]:7.2f}{tag}")
            sys.stdout.flush()
    for name, tot in totals.items():
        default = tot.pop("default")
        ranked = sorted(tot, key=lambda c: tot[c])
        print(f"== {name} (small-message kind): summed per-call time over 128 KiB, 512 KiB and 2 MiB")
        print("   rank  block vec ntl nts wg/cu      us")
        for i, c in enumerate(ranked):
            if i < args.top or c == default:
                tag = "  <- default" if c == default else ""
                print(f"   {i + 1:4d}  {c[0]:5d} {c[1]:3d} {c[2]:3d} {c[3]:3d} {c[4]:5d} {tot[c]:7.2f}{tag}")
    torch.cuda.synchronize()
    if err.cpu().tolist()[0]:
        raise RuntimeError("recursive doubling or unpack saw bad sequence numbers")
    return 0


def crossover(args):
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    blib, vp = _bench_lib()
    sh = torch.cuda.current_stream().cuda_stream
    nbuf = 128 << 20                                  # elements per buffer (256 MiB)
    ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, nbuf, 6, dev)]
    outs = [torch.empty(nbuf, dtype=torch.int16, device=dev) for _ in range(P)]
    ia = (vp * P)(*[t.data_ptr() for t in ins])
    oa = (vp * P)(*[t.data_ptr() for t in outs])
    pairs = {"oneshot": (tar.AR_KERNEL_ONESHOT, tar.AR_KERNEL_ONESHOT_SMALL, 0),
             "2stage": (tar.AR_KERNEL_2STAGE, tar.AR_KERNEL_2STAGE_SMALL, 1),
             "rd": (tar.AR_KERNEL_RD, tar.AR_KERNEL_RD_SMALL, None)}
    sizes = [128 << 10, 512 << 10, 2 << 20, 4 << 20, 8 << 20, 16 << 20, 32 << 20, 64 << 20]
    res = {}
    words = rdo = None
    err = torch.empty(2, dtype=torch.int64, device=dev)
    for name, (kl, ks, which) in pairs.items():
        shapes = {"large": tar.ar_get_launch_shape(kl), "small": tar.ar_get_launch_shape(ks)}
        if name == "rd":
            del ins, outs
            torch.cuda.empty_cache()
            words = [torch.full((nbuf // 2,), 1 << 32, dtype=torch.int64, device=dev) for _ in range(P)]
            rdo = [torch.empty(nbuf // 2, dtype=torch.int64, device=dev) for _ in range(P)]
            wa = (vp * P)(*[t.data_ptr() for t in words])
            ra = (vp * P)(*[t.data_ptr() for t in rdo])
            tar.ar_err_init(err)
        for _ in range(args.rounds):
            for S in sizes:
                n = S // 2
                iters = max(20, min(2000, int(2e5 // (S >> 10))))
                nsets = min(nbuf // n, max(2, (4 << 30) // (16 * S)))
                for label, shp in shapes.items():
                    tar.ar_set_launch_shape(kl, *shp)        # both kinds take the shape under test
                    tar.ar_set_launch_shape(ks, *shp)
                    if which is None:
                        hot = _check_us(blib.arb_decode_us(None, None, wa, ra, P, n, None, 0, err.data_ptr(), 0,
                                                           iters, sh), name)
                        cold = float("nan")
                    else:
                        hot = _check_us(blib.arb_stream_us(which, ia, oa, P, n, None, iters, sh), name)
                        cold = _check_us(blib.arb_stream_rot_us(which, ia, oa, P, n, n, nsets, iters, sh), name)
                    res.setdefault((name, S, label), []).append((hot, cold))
        tar.ar_set_launch_shape(kl, *shapes["large"])
        tar.ar_set_launch_shape(ks, *shapes["small"])
        print(f"[tune] crossover {name} done", file=sys.stderr, flush=True)
        print(f"== {name}: us per call, large-message default {tuple(shapes['large'])} vs small-message default "
              f"{tuple(shapes['small'])}; hot / cold" + (" (RD: bf16 size; payload is twice that)" if which is None else ""))
        print("    size per buffer      large hot   large cold   small hot   small cold   default used")
        for S in sizes:
            lv = res[(name, S, "large")]
            sv = res[(name, S, "small")]
            med = lambda v, i: statistics.median(x[i] for x in v)
            used = "small" if S // 2 <= tar.AR_SMALL_ELEMS else "large"
            print(f"    {S >> 10:10d} KiB {med(lv, 0):12.2f} {med(lv, 1):12.2f} {med(sv, 0):11.2f} "
                  f"{med(sv, 1):12.2f}   {used}")
        sys.stdout.flush()
    torch.cuda.synchronize()
    if err.cpu().tolist()[0]:
        raise RuntimeError("recursive doubling saw bad sequence numbers")
    return 0


if __name__ == "__main__":
    sys.exit(main())
