"""Launch shapes judged over buffer placements.

The bandwidth of the 8-stream kernels depends on where the P rank buffers
sit relative to one another, and the best launch shape for one placement
can lose badly on another.  This sweep times candidate shapes of the
one-shot, fused two-stage, ubatch and fused recursive-doubling kernels, and
of the fp8 quantise and fp8 reduces, on the bench workload (P = 8, bf16
[16384 x 8192] per rank, N(0,1)) with the buffers placed four ways:

* ``separate`` -- one allocation per buffer (as bench.py allocates them);
* ``pow2``     -- one allocation, buffer p at p * (buffer size): a
  power-of-two stride between the P buffers;
* ``skew``     -- one allocation, stride (buffer size + 1 MiB + 4096 elements);
* ``half``     -- the first half of P buffers twice as large (the shape of a
  ubatch split: each ubatch's rows are a part of a larger tensor).

Outputs are placed the same way as inputs (fp8 codes and scale bytes
too).  Each shape is set with
ar_set_launch_shape and timed with HIP events around `reps` back-to-back
calls, in a shuffled order per round; the median over rounds is reported per
placement, with the minimum and the mean over placements.  GB/s counts each
input read once and each output written once (payload words for RD; codes
and scale bytes for fp8).

Usage: python -m tensor_all_reduce_amd.placement [--kinds oneshot,2stage,rd,ubatch,quant,fp8r1,fp8rp]
       [--rounds 3]
"""
from __future__ import annotations

import argparse
import random
import statistics
import sys

import torch

import tensor_all_reduce_amd as tar

P, ROWS, HIDDEN = 8, 16384, 8192
PLACEMENTS = ("separate", "pow2", "skew", "half")
KINDS = {"oneshot": tar.AR_KERNEL_ONESHOT, "2stage": tar.AR_KERNEL_2STAGE, "ubatch": tar.AR_KERNEL_UBATCH,
         "rd": tar.AR_KERNEL_RD, "quant": tar.AR_KERNEL_QUANT_FP8, "fp8r1": tar.AR_KERNEL_REDUCE_FP8,
         "fp8rp": tar.AR_KERNEL_REDUCE_FP8_ALL}
FP8_KINDS = ("quant", "fp8r1", "fp8rp")
# (block, vec, nt_loads, nt_stores, wg_per_cu): the leaders of the single-placement sweeps
SHAPES = {
    "oneshot": [(256, 1, 1, 1, 2), (64, 1, 1, 1, 8), (64, 1, 1, 0, 16), (64, 1, 1, 0, 8), (64, 1, 1, 1, 16),
                (64, 1, 1, 0, 12), (128, 1, 1, 0, 8), (64, 2, 1, 0, 8)],
    "2stage": [(64, 2, 1, 1, 4), (64, 2, 1, 1, 5), (64, 1, 1, 1, 6), (64, 1, 1, 1, 8), (64, 1, 1, 1, 5),
               (64, 1, 1, 1, 4), (128, 1, 1, 1, 4), (64, 2, 1, 1, 3)],
    "ubatch": [(64, 1, 1, 1, 6), (64, 1, 1, 1, 8), (64, 2, 1, 1, 5), (64, 2, 1, 1, 4), (64, 1, 1, 1, 4),
               (64, 1, 1, 1, 5)],
    "rd": [(64, 1, 1, 1, 8), (64, 1, 1, 1, 6), (64, 1, 1, 1, 10), (64, 1, 1, 1, 5), (64, 1, 0, 1, 8),
           (128, 1, 1, 1, 4)],
    "quant": [(64, 2, 1, 1, 0), (64, 1, 1, 1, 0), (128, 2, 1, 1, 0), (256, 1, 1, 1, 0), (64, 2, 1, 0, 0),
              (64, 2, 0, 1, 0), (64, 2, 1, 1, 8), (64, 2, 1, 1, 4), (128, 1, 1, 1, 4)],
    "fp8r1": [(128, 1, 1, 1, 8), (128, 1, 1, 1, 10), (64, 1, 1, 1, 8), (64, 1, 1, 1, 16), (128, 2, 1, 1, 8),
              (128, 1, 1, 1, 4), (256, 1, 1, 1, 4), (128, 1, 1, 0, 8), (128, 1, 1, 1, 0)],
    "fp8rp": [(128, 1, 1, 1, 5), (128, 1, 1, 1, 6), (128, 1, 1, 1, 4), (64, 1, 1, 1, 6), (64, 1, 1, 1, 8),
              (128, 1, 1, 1, 8), (256, 1, 1, 1, 3), (128, 2, 1, 1, 6), (128, 1, 1, 1, 0)],
}


def place(dtype, count: int, how: str, dev):
    """P views of `count` elements each, placed as `how` says."""
    if how == "separate":
        return [torch.empty(count, dtype=dtype, device=dev) for _ in range(P)]
    if how == "pow2":
        big = torch.empty(count * P, dtype=dtype, device=dev)
        return [big[p * count:(p + 1) * count] for p in range(P)]
    if how == "skew":
        stride = count + (1 << 20) // torch.empty(0, dtype=dtype).element_size() + 4096
        big = torch.empty(stride * P, dtype=dtype, device=dev)
        return [big[p * stride:p * stride + count] for p in range(P)]
    if how == "half":
        return [torch.empty(2 * count, dtype=dtype, device=dev)[:count] for _ in range(P)]
    raise ValueError(how)


def time_calls(fn, reps: int) -> float:
    fn()
    fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def sweep(kind_fns, kinds, rounds, reps, how, res, rng):
    for _ in range(rounds):
        for k in kinds:
            nbytes, fn = kind_fns[k]
            order = list(SHAPES[k])
            rng.shuffle(order)
            for sh in order:
                before = tar.ar_get_launch_shape(KINDS[k])
                tar.ar_set_launch_shape(KINDS[k], *sh)
                try:
                    ms = time_calls(fn, reps)
                finally:
                    tar.ar_set_launch_shape(KINDS[k], *before)
                res.setdefault((k, sh, how), []).append(nbytes / ms / 1e6)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--kinds", default="oneshot,2stage,ubatch,rd")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--reps", type=int, default=6)
    args = ap.parse_args(argv)
    kinds = [k for k in args.kinds.split(",") if k]
    for k in kinds:
        if k not in KINDS:
            raise SystemExit(f"unknown kind {k!r}; choose from {', '.join(KINDS)}")
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    tar.lib()
    dev = torch.device("cuda:0")
    n, W = ROWS * HIDDEN, ROWS * HIDDEN // 2
    rng = random.Random(7)
    res = {}
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    for how in PLACEMENTS:
        ins = place(torch.int16, n, how, dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)
        for t in ins:
            t.view(torch.bfloat16).normal_(generator=gen)
        outs = place(torch.int16, n, how, dev)

        def ubatch():
            s0.wait_stream(torch.cuda.current_stream())
            s1.wait_stream(torch.cuda.current_stream())
            tar.ar_reduce_ubatch(ins, outs, ROWS, HIDDEN, 2, None, 1 << 20, tar.AR_VARIANT_2STAGE, streams=[s0, s1])
            torch.cuda.current_stream().wait_stream(s0)
            torch.cuda.current_stream().wait_stream(s1)

        fns = {"oneshot": ((P + 1) * 2 * n, lambda: tar.ar_reduce_oneshot(ins, outs[0])),
               "2stage": (2 * P * 2 * n, lambda: tar.ar_reduce_2stage(ins, outs)),
               "ubatch": (2 * P * 2 * n, ubatch)}
        sweep(fns, [k for k in kinds if k in fns], args.rounds, args.reps, how, res, rng)
        if any(k in FP8_KINDS for k in kinds):
            nb = tar.fp8_scale_count(n)
            codes, scales = place(torch.uint8, n, how, dev), place(torch.uint8, nb, how, dev)
            tar.ar_quantize_fp8(ins, codes, scales)
            fp8_fns = {"quant": (P * (3 * n + nb), lambda: tar.ar_quantize_fp8(ins, codes, scales)),
                       "fp8r1": (P * (n + nb) + 2 * n, lambda: tar.ar_reduce_fp8(codes, scales, outs[:1])),
                       "fp8rp": (P * (n + nb) + P * 2 * n, lambda: tar.ar_reduce_fp8(codes, scales, outs))}
            sweep(fp8_fns, [k for k in kinds if k in FP8_KINDS], args.rounds, args.reps, how, res, rng)
            del codes, scales
        del outs
        torch.cuda.empty_cache()
        if "rd" in kinds:
            words = place(torch.int64, W, how, dev)
            for p in range(P):
                tar.ar_pack_fused(ins[p], words[p], 1)
            del ins
            torch.cuda.empty_cache()
            rdo = place(torch.int64, W, how, dev)
            err = torch.empty(2, dtype=torch.int64, device=dev)
            tar.ar_err_init(err)
            sweep({"rd": (2 * P * 8 * W, lambda: tar.ar_rd_schedule(words, rdo, 1, err))}, ["rd"], args.rounds,
                  args.reps, how, res, rng)
            torch.cuda.synchronize()
            bad = err.cpu().tolist()[0]
            if bad:
                raise SystemExit(f"recursive doubling saw {bad} bad sequence numbers")
            del words, rdo
        else:
            del ins
        torch.cuda.empty_cache()
        print(f"[placement] {how} done", flush=True)
    for k in kinds:
        default = tuple(tar.ar_get_launch_shape(KINDS[k]))
        print(f"== {k}: GB/s per placement (median of {args.rounds} rounds x {args.reps} calls)")
        print("   block vec ntl nts wg/cu " + "".join(f"{h:>10s}" for h in PLACEMENTS) + "       min      mean")
        rows = []
        for sh in SHAPES[k]:
            v = [statistics.median(res[(k, sh, h)]) for h in PLACEMENTS]
            rows.append((statistics.mean(v), sh, v))
        for mean, sh, v in sorted(rows, reverse=True):
            mark = "  <- default" if sh == default else ""
            print(f"   {sh[0]:5d} {sh[1]:3d} {sh[2]:3d} {sh[3]:3d} {sh[4]:5d} " + "".join(f"{x:10.0f}" for x in v)
                  + f"{min(v):10.0f}{mean:10.0f}{mark}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
