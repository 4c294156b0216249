#!/usr/bin/env python3
"""Benchmark of the MI355X all-reduce core (one GPU).

One step = one pass of every hot-path call over one batch: P = 8 simulated
rank buffers of bf16 [16384 x 8192] (the 16k-token prefill hidden state,
256 MiB per buffer), N(0,1) values, and P = 8 buffers of bf16
[16384 x 16384] (512 MiB per buffer) with log-uniform magnitudes in
[2^-8, 2^8] and random signs for the ubatch row, all drawn on the GPU from
seeded generators:

  oneshot   ar_reduce_oneshot            reads 8 buffers, writes 1
  2stage    ar_reduce_2stage (fused)     reads 8, writes 8
  pack      ar_pack_fused x 8            bf16 -> fused payload words (seq s)
  rd        ar_rd_schedule (fused, R1)   3 recursive-doubling steps, 8 payloads
  unpack    ar_unpack_fused x 8          payload -> bf16, seq checked (s + 3)
  ubatch    ar_reduce_ubatch             [16384 x 16384]: 2 ubatches of 8192 rows,
                                         2 streams, 1 MiB chunks, two-stage variant

`value` = credited bytes of the step / step time (GB/s, 1e9 B/s); credited
bytes count each input read once and each output written once (no scratch).
Inputs are resident in HBM before the timed region.

Also reported (not part of `value`): per-call latency of one-shot and
two-stage at 128 KiB / 512 KiB / 2 MiB per buffer (native timing loop, no
Python in the loop), the staged two-stage at the prefill size, the ubatch
reduce's one-shot variant and its two ubatches on one stream, the waiting unpack (on ready payloads
and as a producer -> consumer handoff), attainable copy bandwidth (a plain
copy; eight buffers copied side by side: the 8 -> 8 pattern of the
two-stage, RD and ubatch rows, for the ubatch split over two streams; and
eight buffers gathered into one by XOR: the one-shot's 8 -> 1 pattern), and
the CPU oracle on a bounded sample of the same step (`cpu_baseline`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --ab      A/B of launch shapes and store policies (text report)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0            # MI355X published HBM3E bandwidth, 8 TB/s
P, ROWS, HIDDEN = 8, 16384, 8192
UB_ROWS, UB_HIDDEN = 16384, 16384
CHUNK_BYTES = 1 << 20
METRIC = "achieved HBM GB/s (% of peak) per reduction; µs latency at 128KB–2MB"
# the sources a kernel's counters depend on (code and launch shapes)
KERNEL_SOURCES = ["tensor_all_reduce_amd/csrc/ar_device.hpp", "tensor_all_reduce_amd/csrc/ar_reduce.hip",
                  "tensor_all_reduce_amd/csrc/ar_fused.hip", "tensor_all_reduce_amd/csrc/ar_api.hip"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-cpu-all-cores", action="store_true",
                    help="time the oracle on one core only (skip the all-cores run)")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed steps and the gates (for profiler runs)")
    ap.add_argument("--no-gates", action="store_true",
                    help="skip the per-reduction gate measurements")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calib", action="store_true",
                    help="after the steps, run 3 plain copies of exactly 1 GiB (counter calibration)")
    ap.add_argument("--ab", action="store_true",
                    help="instead of the step: A/B of the launch shapes and store policies of the 8 -> 8 "
                         "and 8 -> 1 kernels and of the ubatch schedule, as a text report")
    ap.add_argument("--ab-small", action="store_true",
                    help="instead of the step: A/B of the small-message kinds' launch shapes at the decode "
                         "sizes, timed inside HIP graphs, as a text report")
    return ap.parse_args()


def sha256_files(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(row: str, sources, path: str | None = None):
    """HBM bytes per launch of a row's kernel from the committed rocprofv3
    counter summary (profiles/traffic_bench_step.txt, "key: value" lines),
    if it was taken on the current kernel sources; else None."""
    if path is None:
        path = os.path.join(ROOT, "profiles", "traffic_bench_step.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != sha256_files(sources):
        return None
    try:
        return float(rec[f"{row}.hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        msg = (f"bench.py measures one GPU only (got --gpus {args.gpus}): the simulated ranks live "
               "in one GPU's HBM and no collective between GPUs is run")
        print(msg, file=sys.stderr)
        print(json.dumps({"error": msg, "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import tensor_all_reduce_amd as tar
    from tensor_all_reduce_amd import synth

    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible")
    tar.lib()                                  # raises if the HIP library is missing
    blib = ctypes.CDLL(os.path.join(ROOT, "tensor_all_reduce_amd", "libarbench.so"))
    vp = ctypes.c_void_p
    blib.arb_stream_us.restype = ctypes.c_double
    blib.arb_stream_us.argtypes = [ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int,
                                   ctypes.c_size_t, vp, ctypes.c_int, vp]
    blib.arb_wall_us.restype = ctypes.c_int
    blib.arb_wall_us.argtypes = [ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int,
                                 ctypes.c_size_t, vp, ctypes.c_int, vp,
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double)]
    blib.arb_enqueue_us.restype = ctypes.c_double
    blib.arb_enqueue_us.argtypes = [ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int,
                                    ctypes.c_size_t, vp, ctypes.c_int, vp]
    blib.arb_copy.restype = ctypes.c_int
    blib.arb_copy.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
    blib.arb_gather_xor.restype = ctypes.c_int
    blib.arb_gather_xor.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                    vp]
    blib.arb_copy_multi.restype = ctypes.c_int
    blib.arb_copy_multi.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_int, vp]
    blib.arb_alu.restype = ctypes.c_int
    blib.arb_alu.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
    blib.arb_stream_rot_us.restype = ctypes.c_double
    blib.arb_stream_rot_us.argtypes = [ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int,
                                       ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp]
    blib.arb_decode_us.restype = ctypes.c_double
    blib.arb_decode_us.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                   ctypes.POINTER(vp), ctypes.c_int, ctypes.c_size_t, vp, ctypes.c_int, vp,
                                   ctypes.c_int, ctypes.c_int, vp]
    blib.arb_handoff_us.restype = ctypes.c_double
    blib.arb_handoff_us.argtypes = [vp, vp, vp, ctypes.c_size_t, ctypes.c_uint32, vp, ctypes.c_int, ctypes.c_int,
                                    vp, vp]
    blib.arb_readsum.restype = ctypes.c_int
    blib.arb_readsum.argtypes = [vp, ctypes.c_size_t, vp, vp]
    blib.arb_consume_chunks.restype = ctypes.c_int
    blib.arb_consume_chunks.argtypes = [vp, ctypes.c_uint32, vp, vp, ctypes.c_size_t, ctypes.c_size_t,
                                        ctypes.c_uint32, ctypes.c_uint32, vp, ctypes.c_int, vp,
                                        ctypes.c_int, vp]

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    main_s = torch.cuda.current_stream()
    n = ROWS * HIDDEN
    B = 2 * n
    W = n // 2

    def e16(m):
        return torch.empty(m, dtype=torch.int16, device=dev)

    def e64(m):
        return torch.empty(m, dtype=torch.int64, device=dev)

    if args.ab_small:
        ab_small_report(tar, torch, synth, dev, main_s)
        return 0

    log(f"device {props.name}, {props.multi_processor_count} CUs; allocating the prefill batch")
    ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, n, 4, dev)]
    out1 = e16(n)
    outs = [e16(n) for _ in range(P)]
    words = [e64(W) for _ in range(P)]
    rdo = [e64(W) for _ in range(P)]
    ux = [e16(n) for _ in range(P)]
    err = e64(2)
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    # the ubatch row's own batch: [16384 x 16384] per rank, log-uniform magnitudes
    n5 = UB_ROWS * UB_HIDDEN
    B5 = 2 * n5
    uin = [t.view(torch.int16) for t in synth.device_rank_buffers("logmag", P, n5, 5, dev)]
    ubo = [e16(n5) for _ in range(P)]

    if args.ab:
        ab_report(args, tar, blib, torch, dev, main_s, ins, outs, out1, uin, ubo, s0, s1)
        return 0

    rows = ["oneshot", "2stage", "pack", "rd", "unpack", "ubatch"]
    credited = {
        "oneshot": (P + 1) * B,
        "2stage": 2 * P * B,
        "pack": P * (B + 2 * B),
        "rd": P * 2 * B * 2,
        "unpack": P * (2 * B + B),
        "ubatch": 2 * P * B5,
    }
    launches = {"oneshot": 1, "2stage": 1, "pack": P, "rd": 1, "unpack": P, "ubatch": 2}
    # the ubatch row's two launches run at the same time on two streams
    concurrent = {"ubatch"}
    kernel_of = {"oneshot": "k_reduce<8,1>", "2stage": "k_reduce<8,8>", "pack": "k_pack",
                 "rd": "k_rd_fused<8,R1>", "unpack": "k_unpack", "ubatch": "k_reduce<8,8> chunked, x2 concurrent"}
    step_bytes = sum(credited.values())

    def run_row(name, seq, uev=None):
        if name == "oneshot":
            tar.ar_reduce_oneshot(ins, out1)
        elif name == "2stage":
            tar.ar_reduce_2stage(ins, outs)
        elif name == "pack":
            for r in range(P):
                tar.ar_pack_fused(ins[r], words[r], seq)
        elif name == "rd":
            tar.ar_err_init(err)
            tar.ar_rd_schedule(words, rdo, seq, err)
        elif name == "unpack":
            for r in range(P):
                tar.ar_unpack_fused(rdo[r], ux[r], seq + 3, err)
        elif name == "ubatch":
            # the two-stream timing protocol: a start event on stream A (s0),
            # ordered after the step's earlier rows, that B (s1) waits on; one
            # ubatch on each; A waits for B's end event and records its own.
            # The row is timed from A's start event to A's end event.
            start, end, b_end = uev if uev is not None else [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            s0.wait_stream(main_s)
            start.record(s0)
            s1.wait_event(start)
            tar.ar_reduce_ubatch(uin, ubo, UB_ROWS, UB_HIDDEN, 2, None, CHUNK_BYTES, tar.AR_VARIANT_2STAGE,
                                 [s0, s1])
            b_end.record(s1)
            s0.wait_event(b_end)
            end.record(s0)
            main_s.wait_stream(s0)

    # ---------------------------------------------------------------- timed steps
    log(f"warmup {args.warmup} steps")
    for w in range(args.warmup):
        for r in rows:
            run_row(r, 1000 + w)
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(rows) + 1)] for _ in range(K)]
    uev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(main_s)
        for i, r in enumerate(rows):
            run_row(r, k + 1, uev[k])
            ev[k][i + 1].record(main_s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev[0][0].elapsed_time(ev[K - 1][len(rows)])
    row_ms = {r: sum(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(K)) / K for i, r in enumerate(rows)}
    # the ubatch row by its own protocol events on stream A (start to end)
    row_ms["ubatch"] = sum(uev[k][0].elapsed_time(uev[k][1]) for k in range(K)) / K
    e = err.cpu().numpy().view(np.uint64)
    assert int(e[0]) == 0, "sequence-number mismatches in the bench step"
    # every output of the step agrees with the one-shot result on device
    for o in outs:
        assert torch.equal(o, out1), "two-stage output differs from one-shot"
    # the ubatch row's outputs agree with the fused two-stage of the same batch
    # (outs of the other batch are reused as scratch for the check)
    chk = [e16(n5) for _ in range(2)]
    tar.ar_reduce_oneshot(uin, chk[0])
    torch.cuda.synchronize()
    for o in ubo:
        assert torch.equal(o, chk[0]), "ubatch output differs from the one-shot of its batch"
    del chk
    ms_per_step = gpu_ms / K
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    step_ms = sorted(ev[k][0].elapsed_time(ev[k][len(rows)]) for k in range(K))
    pct = lambda a, q: a[min(len(a) - 1, int(q * len(a)))]
    log(f"{ms_per_step:.3f} ms/step (wall {1e3 * wall / K:.3f}), {value:.1f} GB/s")

    per_row = {}
    for r in rows:
        gbps = credited[r] / (row_ms[r] * 1e-3) / 1e9
        per_row[r] = {"kernel": kernel_of[r], "launches": launches[r], "ms": round(row_ms[r], 4),
                      "credited_bytes": credited[r], "GBps": round(gbps, 1),
                      "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}
    # the dominant row by time; for a row whose launches run concurrently the
    # rate is the row's bytes over the row's time (both launches together),
    # otherwise bytes per launch over the mean launch time
    dom = max(rows, key=lambda r: row_ms[r])
    if dom in concurrent:
        dom_launch_ms, dom_bytes = row_ms[dom], credited[dom]
    else:
        dom_launch_ms, dom_bytes = row_ms[dom] / launches[dom], credited[dom] / launches[dom]
    achieved = dom_bytes / (dom_launch_ms * 1e-3) / 1e9
    traffic = load_traffic(dom, KERNEL_SOURCES)
    if traffic is not None and dom in concurrent:
        traffic *= launches[dom]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": traffic,
                "kernel": kernel_of[dom], "row": dom, "algorithmic_bytes_per_launch": dom_bytes,
                "avg_launch_ms": round(dom_launch_ms, 4)}
    if dom in concurrent:
        roofline["launches"] = launches[dom]
        roofline["note"] = ("the row's launches run concurrently on two streams: achieved = the row's "
                            "algorithmic bytes / the row's time (both launches together); "
                            "avg_launch_ms is that row time")

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "P=8 simulated ranks; one-shot + fused two-stage + pack + recursive doubling "
                               "+ unpack on bf16 [16384 x 8192] per rank (16k-token prefill hidden state, "
                               "256 MiB/buffer), N(0,1); two-ubatch chunked two-stage reduce on bf16 "
                               "[16384 x 16384] per rank (512 MiB/buffer, 2 streams, 1 MiB chunks), "
                               "log-uniform magnitudes in [2^-8, 2^8]",
                   "P": P, "shape_per_rank": [ROWS, HIDDEN], "ubatch_shape_per_rank": [UB_ROWS, UB_HIDDEN],
                   "accumulate": "f32",
                   "step_credited_bytes": step_bytes, "parallelism": "none (one GPU)"},
        "roofline": roofline,
        "rows": per_row,
        "step_ms_spread": {"p10": round(pct(step_ms, 0.1), 4), "p50": round(pct(step_ms, 0.5), 4),
                           "p90": round(pct(step_ms, 0.9), 4)},
        "kernel_sources_sha256": sha256_files(KERNEL_SOURCES),
    }

    if not args.no_gates:
        result["gates"] = gates(tar, torch, main_s, ins, outs, uin, ubo, s0, s1)

    if args.copy_calib:
        cb = 1 << 30
        src = torch.empty(cb // 2, dtype=torch.int16, device=dev)
        dst = torch.empty(cb // 2, dtype=torch.int16, device=dev)
        src.fill_(1)
        for _ in range(3):
            if blib.arb_copy(src.data_ptr(), dst.data_ptr(), cb, 64, main_s.cuda_stream) != 0:
                raise RuntimeError("arb_copy failed")
        torch.cuda.synchronize()
        result["copy_calib_bytes"] = cb
        del src, dst

    if not args.no_extras:
        result.update(extras(args, tar, blib, torch, np, dev, main_s, ins, outs, out1, e16, s0, s1, uin, ubo))
        del ins, outs, words, rdo, ux, ubo, out1, uin
        torch.cuda.empty_cache()
        # the same rates against the attainable bandwidth measured in this run
        for r in rows:
            per_row[r]["frac_of_copy"] = round(per_row[r]["GBps"] / result["copy_GBps"], 4)
        # the one-shot, two-stage, RD and ubatch rows against a plain copy with
        # the same access pattern: 8 -> 1 for the one-shot; 8 -> 8 on one
        # stream over whole buffers, or on two over the halves, for the others
        for r, ref in (("oneshot", "copy_8to1_GBps"), ("2stage", "copy_8to8_GBps"), ("rd", "copy_8to8_GBps"),
                       ("ubatch", "copy_8to8_two_streams_GBps")):
            per_row[r]["frac_of_pattern_copy"] = round(per_row[r]["GBps"] / result[ref], 4)
        roofline["frac_of_copy"] = round(achieved / result["copy_GBps"], 4)
        pattern = {"oneshot": "copy_8to1_GBps", "ubatch": "copy_8to8_two_streams_GBps"}.get(dom, "copy_8to8_GBps")
        roofline["frac_of_pattern_copy"] = round(achieved / result[pattern], 4)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args, np)
    print(json.dumps(result), flush=True)
    return 0


def gates(tar, torch, main_s, ins, outs, uin, ubo, s0, s1):
    """The per-reduction targets, timed as throughput: after 20 warm-up
    calls, HIP events bracket K back-to-back calls (K sized so a bracket
    lasts at least 100 ms), 30 brackets, median of time / K with p10 / p90.
    GB/s counts each input read once and each output written once.

      c4_2stage_fused  P=8 [16384 x 8192], ar_reduce_2stage (fused):
                       >= 80% of 8 TB/s means <= 671 us per call
      c5_ubatch        P=8 [16384 x 16384], ar_reduce_ubatch, two-stage, two
                       8192-row ubatches on two streams, 1 MiB chunks:
                       <= 1.342 ms per call; each call by the two-stream
                       protocol (a start event on stream A that B waits on,
                       one ubatch on each, A waits for B's end), the
                       bracket's events on A
      c4_oneshot       ar_reduce_oneshot (no target), writing the P output
                       buffers in turn: its 256 MiB output would otherwise
                       stay in the 256 MiB last-level cache between calls
                       and never pay its write-back"""
    def bracket(fn, brackets=30, target_ms=100.0, st=None):
        st = main_s if st is None else st          # the stream the bracket's events are recorded on
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(10):
            fn()
        e1.record(st)
        e1.synchronize()
        k = max(10, int(target_ms / max(e0.elapsed_time(e1) / 10, 1e-3)) + 1)
        per = []
        for _ in range(brackets):
            e0.record(st)
            for _ in range(k):
                fn()
            e1.record(st)
            e1.synchronize()
            per.append(e0.elapsed_time(e1) / k * 1e3)
        per.sort()
        return per[len(per) // 2], per[len(per) // 10], per[(len(per) * 9) // 10], k

    n, n5 = ROWS * HIDDEN, UB_ROWS * UB_HIDDEN
    turn = [0]

    def oneshot():
        turn[0] += 1
        tar.ar_reduce_oneshot(ins, outs[turn[0] % P])

    # the two-stream timing protocol, per call: a start event on stream A
    # (s0) that B (s1) waits on, one ubatch on each, A waits for B's end; the
    # bracket's own events are on A
    u_start, u_bend = torch.cuda.Event(), torch.cuda.Event()

    def ubatch():
        u_start.record(s0)
        s1.wait_event(u_start)
        tar.ar_reduce_ubatch(uin, ubo, UB_ROWS, UB_HIDDEN, 2, None, CHUNK_BYTES, tar.AR_VARIANT_2STAGE, [s0, s1])
        u_bend.record(s1)
        s0.wait_event(u_bend)

    s0.wait_stream(main_s)
    cases = (("c4_2stage_fused", lambda: tar.ar_reduce_2stage(ins, outs), 2 * P * 2 * n, main_s),
             ("c5_ubatch", ubatch, 2 * P * 2 * n5, s0),
             ("c4_oneshot", oneshot, (P + 1) * 2 * n, main_s))
    res = {}
    for name, fn, cred, st in cases:
        med, p10, p90, k = bracket(fn, st=st)
        main_s.wait_stream(s0)
        gbps = cred / (med * 1e-6) / 1e9
        res[name] = {"us": round(med, 2), "us_p10": round(p10, 2), "us_p90": round(p90, 2), "calls_per_bracket": k,
                     "brackets": 30, "credited_bytes": cred, "GBps": round(gbps, 1),
                     "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        if name != "c4_oneshot":
            target_us = cred / (0.8 * PEAK_HBM_GBPS * 1e9) * 1e6
            res[name]["target_us"] = round(target_us, 1)
            res[name]["met"] = bool(med <= target_us)
        log(f"gate {name}: {med:.1f} us (p10 {p10:.1f}, p90 {p90:.1f}), {gbps:.0f} GB/s, "
            f"{gbps / PEAK_HBM_GBPS:.4f} of peak")
    return res


def extras(args, tar, blib, torch, np, dev, main_s, ins, outs, out1, e16, s0, s1, uin, ubo):
    vp = ctypes.c_void_p
    sh = main_s.cuda_stream
    res = {}

    def parr(ts):
        a = (vp * len(ts))()
        for i, t in enumerate(ts):
            a[i] = t.data_ptr()
        return a

    # staged two-stage at the prefill size (scratch round trip not credited)
    n = ROWS * HIDDEN
    scratch = e16(n)
    us = blib.arb_stream_us(2, parr(ins), parr(outs), P, n, scratch.data_ptr(), 20, sh)
    res["2stage_staged_prefill"] = {"us": round(us, 2),
                                    "GBps_credited": round(2 * P * 2 * n / (us * 1e-6) / 1e9, 1)}
    us = blib.arb_stream_us(1, parr(ins), parr(outs), P, n, None, 20, sh)
    res["2stage_fused_prefill"] = {"us": round(us, 2),
                                   "GBps_credited": round(2 * P * 2 * n / (us * 1e-6) / 1e9, 1),
                                   "frac_of_peak": round(2 * P * 2 * n / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
    del scratch
    log("prefill staged/fused two-stage timed")

    # attainable bandwidth: plain copy of 2 GiB
    cb = 1 << 31
    src = torch.empty(cb // 2, dtype=torch.int16, device=dev)
    dst = torch.empty(cb // 2, dtype=torch.int16, device=dev)
    src.fill_(1)
    best = 0.0
    for block in (64, 128, 256):
        for _ in range(3):
            blib.arb_copy(src.data_ptr(), dst.data_ptr(), cb, block, sh)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main_s)
        for _ in range(10):
            blib.arb_copy(src.data_ptr(), dst.data_ptr(), cb, block, sh)
        e1.record(main_s)
        torch.cuda.synchronize()
        gbps = 2 * cb * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        best = max(best, gbps)
    res["copy_GBps"] = round(best, 1)
    # attainable bandwidth of the 8 -> 8 pattern itself: eight 256 MiB buffers
    # copied side by side into eight others (16 concurrent streams, no
    # arithmetic), best over groups per lane and the workgroups-per-CU cap
    best8, shape8 = 0.0, None
    for vec in (1, 2):
        for wg in (0, 2, 3, 4, 5, 6, 8):
            for _ in range(2):
                if blib.arb_copy_multi(parr(ins), parr(outs), P, 2 * n, vec, wg, sh) != 0:
                    raise RuntimeError("arb_copy_multi failed")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(main_s)
            for _ in range(8):
                blib.arb_copy_multi(parr(ins), parr(outs), P, 2 * n, vec, wg, sh)
            e1.record(main_s)
            torch.cuda.synchronize()
            gbps = 2 * P * 2 * n * 8 / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if gbps > best8:
                best8, shape8 = gbps, {"vec": vec, "wg_per_cu": wg}
    res["copy_8to8_GBps"] = round(best8, 1)
    res["copy_8to8_shape"] = shape8
    # the one-shot row's pattern: eight 256 MiB buffers read, their XOR
    # written to one output (the one-shot's tiling, no float arithmetic),
    # best over store kind and the workgroups-per-CU cap.  The output rotates
    # over the P output buffers, as the one-shot gate's does: rewriting one
    # output call after call would leave part of it in the 256 MiB last-level
    # cache, a write-back the step's one-shot (behind five other rows) pays
    best1, shape1 = 0.0, None
    for nts in (0, 1):
        for wg in (0, 4, 8, 12, 16):
            for i in range(2):
                if blib.arb_gather_xor(parr(ins), P, outs[i % P].data_ptr(), 2 * n, nts, wg, sh) != 0:
                    raise RuntimeError("arb_gather_xor failed")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(main_s)
            for i in range(8):
                blib.arb_gather_xor(parr(ins), P, outs[(i + 2) % P].data_ptr(), 2 * n, nts, wg, sh)
            e1.record(main_s)
            torch.cuda.synchronize()
            gbps = (P + 1) * 2 * n * 8 / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if gbps > best1:
                best1, shape1 = gbps, {"nt_stores": nts, "wg_per_cu": wg}
    res["copy_8to1_GBps"] = round(best1, 1)
    res["copy_8to1_shape"] = shape1
    # the ubatch row's pattern: its own [16384 x 16384] buffers copied 8 -> 8
    # with no arithmetic, split at the middle row, the two halves on two
    # streams at once (as the two ubatch reduces run), on the ubatch streams
    # themselves: HIP maps a process's streams onto a few hardware queues, and
    # two more streams here could put the later producer / consumer pair on
    # one queue, where they would run in turn
    n5 = UB_ROWS * UB_HIDDEN
    h = n5 // 2
    halves = [(parr([x[:h] for x in uin]), parr([o[:h] for o in ubo])),
              (parr([x[h:] for x in uin]), parr([o[h:] for o in ubo]))]

    # timed by the same two-stream protocol as the ubatch row: per call a
    # start event on s0 that s1 waits on, one half on each, s0 waits for s1's
    # end; the bracket's events on s0
    c_start, c_bend = torch.cuda.Event(), torch.cuda.Event()

    def two_streams(vec, wg):
        c_start.record(s0)
        s1.wait_event(c_start)
        for (pi, po), st in zip(halves, (s0, s1)):
            if blib.arb_copy_multi(pi, po, P, 2 * h, vec, wg, st.cuda_stream) != 0:
                raise RuntimeError("arb_copy_multi failed")
        c_bend.record(s1)
        s0.wait_event(c_bend)

    best2, shape2 = 0.0, None
    s0.wait_stream(main_s)
    for vec in (1, 2):
        for wg in (4, 5, 6, 8):
            for _ in range(2):
                two_streams(vec, wg)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s0)
            for _ in range(8):
                two_streams(vec, wg)
            e1.record(s0)
            torch.cuda.synchronize()
            gbps = 2 * P * 2 * n5 * 8 / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if gbps > best2:
                best2, shape2 = gbps, {"vec": vec, "wg_per_cu": wg}
    main_s.wait_stream(s0)
    res["copy_8to8_two_streams_GBps"] = round(best2, 1)
    res["copy_8to8_two_streams_shape"] = shape2
    # attainable read bandwidth: read-only sweep of the same 2 GiB
    sink = torch.empty(cb // 16384 + 1, dtype=torch.int32, device=dev)
    for _ in range(3):
        if blib.arb_readsum(src.data_ptr(), cb, sink.data_ptr(), sh) != 0:
            raise RuntimeError("arb_readsum failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(main_s)
    for _ in range(10):
        blib.arb_readsum(src.data_ptr(), cb, sink.data_ptr(), sh)
    e1.record(main_s)
    torch.cuda.synchronize()
    res["read_GBps"] = round(cb * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst, sink
    log(f"copy bandwidth {best:.0f} GB/s, 8 -> 8 copy {best8:.0f} GB/s (two streams over halves {best2:.0f}), "
        f"read-only {res['read_GBps']:.0f} GB/s")

    # latency at decode sizes: P = 2 at one token ([1 x 8192], 16 KiB), then
    # P = 8 at 128 KiB .. 2 MiB per buffer
    lat = {}
    m = HIDDEN
    xi = [x[:m] for x in ins[:2]]
    xo = [o[:m] for o in outs[:2]]
    us = blib.arb_stream_us(0, parr(xi), parr(xo), 2, m, None, 10000, sh)
    p50, p10, p90 = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    if blib.arb_wall_us(0, parr(xi), parr(xo), 2, m, None, 10000, sh, ctypes.byref(p50), ctypes.byref(p10),
                        ctypes.byref(p90)) != 0:
        raise RuntimeError("arb_wall_us failed")
    lat["P2_16KiB"] = {"oneshot": {"stream_us": round(us, 2), "wall_us_p50": round(p50.value, 2),
                                   "wall_us_p90": round(p90.value, 2)}}
    for T in (8, 32, 128):
        m = T * HIDDEN
        xi = [x[:m] for x in ins]
        xo = [o[:m] for o in outs]
        sc = e16(m)
        xb = [x.clone() for x in xi]   # the in-place call's buffers (only timed: their values grow)
        key = f"{2 * m // 1024}KiB"
        lat[key] = {}
        for which, name, bi, bo in ((0, "oneshot", xi, xo), (1, "2stage_fused", xi, xo),
                                    (1, "2stage_fused_inplace", xb, xb), (2, "2stage_staged", xi, xo)):
            us = blib.arb_stream_us(which, parr(bi), parr(bo), P, m, sc.data_ptr(), 10000, sh)
            p50, p10, p90 = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
            rc = blib.arb_wall_us(which, parr(bi), parr(bo), P, m, sc.data_ptr(), 10000, sh,
                                  ctypes.byref(p50), ctypes.byref(p10), ctypes.byref(p90))
            if rc != 0:
                raise RuntimeError(f"arb_wall_us failed: {rc}")
            cred = (P + 1) * 2 * m if which == 0 else 2 * P * 2 * m
            enq = blib.arb_enqueue_us(which, parr(bi), parr(bo), P, m, sc.data_ptr(), 5000, sh)
            if enq < 0:
                raise RuntimeError(f"arb_enqueue_us failed: {enq}")
            lat[key][name] = {"stream_us": round(us, 2), "wall_us_p50": round(p50.value, 2),
                              "wall_us_p90": round(p90.value, 2), "host_enqueue_us": round(enq, 2),
                              "GBps_hot": round(cred / (us * 1e-6) / 1e9, 1)}
    # host cost of a launch itself: empty kernels with no, 8 or 192 bytes of
    # arguments.  HIP enqueues a kernel whose argument segment is at most 112
    # bytes faster; the decode-size one-shot, in-place fused two-stage, pack
    # and unpack kernels take 28-80 bytes and no hidden arguments, the others
    # about 300-440 bytes
    lat["empty_kernel_host_enqueue_us"] = {
        k: round(blib.arb_enqueue_us(w, None, None, 0, 0, None, 5000, sh), 2)
        for k, w in (("no_arguments", -1), ("8_byte_argument", -2), ("192_byte_argument", -3))}
    # the same enqueue with this thread pinned to each core it may use, in
    # turn: on a virtual machine the cost depends on which virtual core the
    # launching thread runs on, so one unpinned figure can land anywhere in
    # this range
    m = 8 * HIDDEN
    xi, xo = [x[:m] for x in ins], [o[:m] for o in outs]
    allowed = sorted(os.sched_getaffinity(0))
    per_core = {}
    try:
        for c in allowed:
            os.sched_setaffinity(0, {c})
            per_core[c] = (blib.arb_enqueue_us(-3, None, None, 0, 0, None, 2000, sh),
                           blib.arb_enqueue_us(0, parr(xi), parr(xo), P, m, None, 2000, sh))
    finally:
        os.sched_setaffinity(0, allowed)
    if any(v < 0 for pair in per_core.values() for v in pair):
        raise RuntimeError("arb_enqueue_us failed")

    def spread(vals):
        vals = sorted(vals)
        return {"min": round(vals[0], 2), "median": round(vals[len(vals) // 2], 2), "max": round(vals[-1], 2)}
    fastest = min(per_core, key=lambda c: per_core[c][1])
    lat["host_enqueue_us_by_core"] = {
        "cores": len(per_core), "fastest_core": fastest,
        "empty_kernel_192_byte_argument": spread(v[0] for v in per_core.values()),
        "oneshot_128KiB": spread(v[1] for v in per_core.values())}

    # the 128 KiB fused two-stage called from Python on the current stream:
    # through the wrapper, whose checks and marshalling run on every call,
    # and through a handle from tar.prepare, marshalled once; host time per
    # call over a loop of calls, and the stream time of the same loop
    def py_loop(fn, k=3000):
        for _ in range(300):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main_s)
        t0 = time.perf_counter()
        for _ in range(k):
            fn()
        t1 = time.perf_counter()
        e1.record(main_s)
        torch.cuda.synchronize()
        return round((t1 - t0) / k * 1e6, 2), round(e0.elapsed_time(e1) * 1e3 / k, 2)

    h2 = tar.prepare(tar.ar_reduce_2stage, xi, xo)
    wh, ws = py_loop(lambda: tar.ar_reduce_2stage(xi, xo))
    ph, ps = py_loop(h2)
    lat["python_binding_128KiB_2stage_fused"] = {"wrapper_host_us": wh, "wrapper_stream_us": ws,
                                                 "prepared_host_us": ph, "prepared_stream_us": ps}
    del h2
    res["latency"] = lat
    log(f"latency measured; from Python at 128 KiB: wrapper {wh} us host / {ws} us stream per call, "
        f"prepared {ph} / {ps}")

    # the same sizes cold: call k uses the (k mod sets)-th disjoint slice of
    # the prefill buffers, at least 64 sets and at least 1 GiB in all (four
    # times the 256 MiB last-level cache), so every call reads and writes HBM
    cold = {}
    for T in (8, 32, 128):
        m = T * HIDDEN
        sets = min(n // m, max(64, -(-(1 << 30) // (2 * P * 2 * m))))
        key = f"{2 * m // 1024}KiB"
        cold[key] = {"sets": sets}
        for which, name in ((0, "oneshot"), (1, "2stage_fused")):
            us = blib.arb_stream_rot_us(which, parr(ins), parr(outs), P, m, m, sets, 4 * sets, sh)
            if us < 0:
                raise RuntimeError(f"arb_stream_rot_us failed: {us}")
            cred = (P + 1) * 2 * m if which == 0 else 2 * P * 2 * m
            cold[key][name] = {"stream_us": round(us, 2), "GBps": round(cred / (us * 1e-6) / 1e9, 1)}
    res["latency_cold"] = cold
    log("cold latency measured")

    # decode all-reduce on fused payloads at [128 x 8192] per rank, P = 8:
    # recursive doubling alone, and the whole chain (P packs, error reset,
    # recursive doubling, P unpacks), seq0 = 1
    def e64(k):
        return torch.empty(k, dtype=torch.int64, device=dev)

    m = 128 * HIDDEN
    xi = [x[:m] for x in ins]
    yo = [o[:m] for o in outs]
    win = [e64(m // 2) for _ in range(P)]
    wout = [e64(m // 2) for _ in range(P)]
    mbox = e64(tar.rd_mailbox_words(P, m))
    derr = e64(2)
    tar.ar_err_init(derr, stream=main_s)
    for p in range(P):
        tar.ar_pack_fused(xi[p], win[p], 1, stream=main_s)
    dec = {}
    for name, mb, flags, chain in (("rd_fused_R1", None, 0, 0), ("rd_fused_R2", None, tar.AR_RD_FP32_CARRY, 0),
                                   ("rd_staged_R1", mbox, tar.AR_RD_STAGED, 0),
                                   ("chain_fused_R1", None, 0, 1), ("chain_staged_R1", mbox, tar.AR_RD_STAGED, 1)):
        us = blib.arb_decode_us(parr(xi), parr(yo), parr(win), parr(wout), P, m,
                                mb.data_ptr() if mb is not None else None, flags, derr.data_ptr(), chain, 2000, sh)
        if us < 0:
            raise RuntimeError(f"arb_decode_us failed: {us}")
        dec[name] = {"stream_us": round(us, 2)}
    torch.cuda.synchronize()
    e = derr.cpu().tolist()
    if e[0] != 0:
        raise RuntimeError(f"decode chain saw {e[0]} bad sequence numbers")
    # the whole chain captured in a HIP graph (20 chains per graph, every
    # chain packs with seq0 = 1, so each replay checks its own sequence
    # numbers): the chain's GPU time without the 2P + 2 host launches
    gside = torch.cuda.Stream()
    gside.wait_stream(main_s)

    def chain(st, staged):
        for p in range(P):
            tar.ar_pack_fused(xi[p], win[p], 1, stream=st)
        tar.ar_err_init(derr, stream=st)
        if staged:
            tar.ar_rd_schedule(win, wout, 1, derr, mailbox=mbox, flags=tar.AR_RD_STAGED, stream=st)
        else:
            tar.ar_rd_schedule(win, wout, 1, derr, stream=st)
        for p in range(P):
            tar.ar_unpack_fused(wout[p], yo[p], 1 + 3, derr, stream=st)

    for name, staged in (("chain_fused_R1", False), ("chain_staged_R1", True)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gside):
            chain(gside, staged)
            gside.synchronize()
            ref = [y.clone() for y in yo]
            with torch.cuda.graph(g, stream=gside):
                for _ in range(20):
                    chain(gside, staged)
        torch.cuda.synchronize()
        for _ in range(3):
            for y in yo:
                y.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(y, r) for y, r in zip(yo, ref)):
                raise RuntimeError(f"{name}: a graph replay differs from the eager chain")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(main_s)
        for _ in range(10):
            g.replay()
        e1.record(main_s)
        torch.cuda.synchronize()
        dec[name]["hip_graph_us"] = round(e0.elapsed_time(e1) * 1e3 / 200, 2)
        bad = int(derr[0].item())
        if bad or not all(torch.equal(y, r) for y, r in zip(yo, ref)):
            raise RuntimeError(f"{name}: the graph's last chain saw {bad} bad sequence numbers or wrong data")
        del g, ref
    res["decode_fused_payload_128x8192"] = dec
    del win, wout, mbox
    log("decode chain measured")

    # the same calls captured in one HIP graph (100 calls per graph), which
    # removes the per-launch host cost from each call
    glat = {}
    side = torch.cuda.Stream()
    side.wait_stream(main_s)
    for T in (8, 32, 128):
        m = T * HIDDEN
        xi = [x[:m] for x in ins]
        xo = [o[:m] for o in outs]
        key = f"{2 * m // 1024}KiB"
        glat[key] = {}
        xb = [x.clone() for x in xi]   # the in-place call's buffers (only timed: their values grow)
        calls = {"oneshot": lambda: tar.ar_reduce_oneshot(xi, xo[0], stream=side),
                 "2stage_fused": lambda: tar.ar_reduce_2stage(xi, xo, stream=side),
                 "2stage_fused_inplace": lambda: tar.ar_reduce_2stage(xb, xb, stream=side)}
        for name, call in calls.items():
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                call()
                side.synchronize()
                with torch.cuda.graph(g, stream=side):
                    for _ in range(100):
                        call()
            torch.cuda.synchronize()
            for _ in range(3):
                g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(main_s)
            for _ in range(20):
                g.replay()
            e1.record(main_s)
            torch.cuda.synchronize()
            glat[key][name] = {"us_per_call": round(e0.elapsed_time(e1) * 1e3 / 2000, 2)}
            del g
        del xb
    # the floor of one graph node on this machine: the same capture of a
    # one-workgroup kernel (torch's fill of 64 floats)
    tiny = torch.zeros(64, dtype=torch.float32, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        tiny.fill_(1.0)
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            for _ in range(100):
                tiny.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(main_s)
    for _ in range(20):
        g.replay()
    e1.record(main_s)
    torch.cuda.synchronize()
    glat["node_floor_one_workgroup_us"] = round(e0.elapsed_time(e1) * 1e3 / 2000, 2)
    del g
    res["latency_hip_graph"] = glat
    log("graph latency measured")

    res.update(overlap(tar, blib, torch, dev, main_s, ins, outs, s0, s1))
    res.update(wait_receive(tar, blib, torch, dev, main_s, ins, outs, s0, s1))
    res.update(fp8(tar, torch, dev, main_s, ins, outs))

    # the ubatch reduce's variants at the row's shape: the one-shot variant
    # (one output, (P + 1) B credited) on two streams, and the two-stage
    # variant with both ubatches on one stream (no overlap between them)
    m = UB_ROWS * UB_HIDDEN
    reps = 10

    def ub_timed(variant, streams, nout):
        # the two-stream protocol as in the step (start event on A that B
        # waits on, A waits for B's end), the bracket's events on A
        a, b = streams
        start, b_end = torch.cuda.Event(), torch.cuda.Event()

        def go():
            if b is not a:
                start.record(a)
                b.wait_event(start)
            tar.ar_reduce_ubatch(uin, ubo[:nout], UB_ROWS, UB_HIDDEN, 2, None, CHUNK_BYTES, variant, streams)
            if b is not a:
                b_end.record(b)
                a.wait_event(b_end)
        a.wait_stream(main_s)
        for _ in range(3):
            go()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(a)
        for _ in range(reps):
            go()
        e1.record(a)
        torch.cuda.synchronize()
        main_s.wait_stream(a)
        return e0.elapsed_time(e1) / reps

    ms = ub_timed(tar.AR_VARIANT_ONESHOT, [s0, s1], 1)
    gbps = (P + 1) * 2 * m / (ms * 1e-3) / 1e9
    res["ubatch_16384x16384_oneshot"] = {"ms": round(ms, 4), "GBps_credited": round(gbps, 1),
                                         "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}
    log(f"ubatch one-shot [16384x16384]: {ms:.3f} ms, {gbps:.0f} GB/s")
    ms = ub_timed(tar.AR_VARIANT_2STAGE, [s0, s0], P)
    gbps = 2 * P * 2 * m / (ms * 1e-3) / 1e9
    res["ubatch_16384x16384_one_stream"] = {"ms": round(ms, 4), "GBps_credited": round(gbps, 1),
                                            "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
                                            "note": "both ubatches on one stream, one after the other"}
    log(f"ubatch [16384x16384] on one stream: {ms:.3f} ms, {gbps:.0f} GB/s")
    torch.cuda.empty_cache()
    return res


def ab_report(args, tar, blib, torch, dev, main_s, ins, outs, out1, uin, ubo, s0, s1):
    """A/B of launch choices on the bench's own buffers, printed as text.

    For the one-shot (8 -> 1), the fused two-stage (8 -> 8), the fused
    recursive doubling and the two-stream ubatch reduce, every candidate shape
    (block, vec, nt_loads, stores, wg_per_cu; stores 1 = non-temporal,
    2 = SC1 write-through, 3 = SC1 + non-temporal) is set with
    ar_set_launch_shape and timed with HIP events around `reps` calls;
    candidates are visited in a shuffled order each round and the median over
    rounds is reported, so slow drift of the device affects all alike.  Then
    the bounded ubatch grid's footprint is timed alone and beside a bf16 GEMM
    on another stream, and last the 8 -> 8 kernels over buffer placements
    (placement_report).  The one-shot writes its output to the P output
    buffers in turn: its 256 MiB
    output fits the 256 MiB last-level cache, and calls that rewrite one
    buffer leave it there without ever paying its write-back to HBM.  The
    ubatch schedule is also run with both ubatches on one stream.  Reference
    rows time plain copies with each kernel's access pattern (no arithmetic).
    GB/s counts each input read once and each output written once."""
    import itertools
    import random
    import statistics

    n = ROWS * HIDDEN
    n5 = UB_ROWS * UB_HIDDEN
    B, B5 = 2 * n, 2 * n5
    W = n // 2
    words = [torch.empty(W, dtype=torch.int64, device=dev) for _ in range(P)]
    rdo = [torch.empty(W, dtype=torch.int64, device=dev) for _ in range(P)]
    err = torch.empty(2, dtype=torch.int64, device=dev)
    for r in range(P):
        tar.ar_pack_fused(ins[r], words[r], 1)
    tar.ar_err_init(err)
    vp = ctypes.c_void_p

    def parr(ts):
        a = (vp * len(ts))()
        for i, t in enumerate(ts):
            a[i] = t.data_ptr()
        return a

    # two-stream calls follow the timing protocol: a start event on stream A
    # (s0) that B waits on, one ubatch on each, A waits for B's end; they are
    # timed on A (time_calls(fn, s0))
    u_start, u_bend = torch.cuda.Event(), torch.cuda.Event()

    def ubatch(streams):
        a, b = streams
        if b is not a:
            u_start.record(a)
            b.wait_event(u_start)
        tar.ar_reduce_ubatch(uin, ubo, UB_ROWS, UB_HIDDEN, 2, None, CHUNK_BYTES, tar.AR_VARIANT_2STAGE, streams)
        if b is not a:
            u_bend.record(b)
            a.wait_event(u_bend)

    turn = [0]

    def oneshot_rotating():
        turn[0] += 1
        tar.ar_reduce_oneshot(ins, outs[turn[0] % P])

    kinds = {
        "oneshot": (tar.AR_KERNEL_ONESHOT, (P + 1) * B, oneshot_rotating,
                    list(itertools.product((64, 128), (1,), (1,), (0, 1, 2, 3), (0, 8, 12, 16)))),
        "2stage": (tar.AR_KERNEL_2STAGE, 2 * P * B, lambda: tar.ar_reduce_2stage(ins, outs),
                   list(itertools.product((64,), (1, 2), (1,), (0, 1, 2, 3), (4, 5, 6, 8)))),
        "rd": (tar.AR_KERNEL_RD, 4 * P * B, lambda: tar.ar_rd_schedule(words, rdo, 1, err),
               list(itertools.product((64,), (1,), (1,), (0, 1, 2, 3), (6, 8, 10)))),
        "ubatch_two_streams": (tar.AR_KERNEL_UBATCH, 2 * P * B5, lambda: ubatch([s0, s1]),
                               list(itertools.product((64,), (1,), (1,), (1, 3), (3, 4, 6, 8))), s0),
        "ubatch_one_stream": (tar.AR_KERNEL_UBATCH, 2 * P * B5, lambda: ubatch([s0, s0]),
                              list(itertools.product((64,), (1,), (1,), (1, 3), (3, 4, 6, 8))), s0),
    }
    reps, rounds = 4, 3
    rng = random.Random(11)

    def time_calls(fn, st=None):
        # events on `st` (default the launch stream); a stream other than the
        # launch stream takes over from it, and hands back, outside the timing
        st = main_s if st is None else st
        if st is not main_s:
            st.wait_stream(main_s)
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        e1.synchronize()
        if st is not main_s:
            main_s.wait_stream(st)
        return e0.elapsed_time(e1) / reps

    print("# A/B of launch shapes on the bench buffers: P=8, bf16 [16384 x 8192] per rank "
          "([16384 x 16384] for the ubatch rows)")
    print(f"# command: python bench.py --ab   ({rounds} shuffled rounds x {reps} calls, median per candidate)")
    print(f"# device: {torch.cuda.get_device_properties(dev).name}, "
          f"{torch.cuda.get_device_properties(dev).multi_processor_count} CUs")
    for name, spec in kinds.items():
        kind, cred, fn, cands = spec[:4]
        tst = spec[4] if len(spec) > 4 else None
        default = tar.ar_get_launch_shape(kind)
        if default not in cands:
            cands = cands + [default]
        times = {c: [] for c in cands}
        for _ in range(rounds):
            order = cands[:]
            rng.shuffle(order)
            for c in order:
                tar.ar_set_launch_shape(kind, *c)
                times[c].append(time_calls(fn, tst))
        tar.ar_set_launch_shape(kind, *default)
        med = {c: statistics.median(v) for c, v in times.items()}
        ranked = sorted(cands, key=lambda c: med[c])
        best = med[ranked[0]]
        print(f"== {name}: {cred} algorithmic bytes per call, {len(cands)} shapes")
        print("   block vec ntl stores wg/cu        ms      GB/s  frac-of-8TB/s  vs-best")
        for c in ranked:
            gbps = cred / (med[c] * 1e-3) / 1e9
            tag = "  <- default" if c == default else ""
            print(f"   {c[0]:5d} {c[1]:3d} {c[2]:3d} {c[3]:6d} {c[4]:5d} {med[c]:9.4f} {gbps:9.1f}  "
                  f"{gbps / PEAK_HBM_GBPS:13.4f}  {best / med[c]:7.4f}{tag}")
        sys.stdout.flush()
        log(f"ab: {name} done")
    # references: the same access patterns copied with no arithmetic
    print("== reference copies (no arithmetic), best over the listed shapes")

    def best_of(fn_by_shape, shapes, cred, st=None):
        out = []
        for sh in shapes:
            out.append((time_calls(lambda: fn_by_shape(sh), st), sh))
        t, sh = min(out)
        return cred / (t * 1e-3) / 1e9, sh

    def copy8(sh):
        if blib.arb_copy_multi(parr(ins), parr(outs), P, B, sh[0], sh[1], main_s.cuda_stream) != 0:
            raise RuntimeError("arb_copy_multi failed")

    gturn = [0]

    def gather(sh):   # the output rotates over the P outputs, as the one-shot candidates' do
        gturn[0] += 1
        if blib.arb_gather_xor(parr(ins), P, outs[gturn[0] % P].data_ptr(), B, sh[0], sh[1],
                               main_s.cuda_stream) != 0:
            raise RuntimeError("arb_gather_xor failed")

    h = n5 // 2
    halves = [(parr([x[:h] for x in uin]), parr([o[:h] for o in ubo])),
              (parr([x[h:] for x in uin]), parr([o[h:] for o in ubo]))]

    def copy_two(sh):
        u_start.record(s0)
        s1.wait_event(u_start)
        for (pi, po), st in zip(halves, (s0, s1)):
            if blib.arb_copy_multi(pi, po, P, 2 * h, sh[0], sh[1], st.cuda_stream) != 0:
                raise RuntimeError("arb_copy_multi failed")
        u_bend.record(s1)
        s0.wait_event(u_bend)

    caps = (0, 4, 5, 6, 8)
    g, sh = best_of(copy8, [(v, w) for v in (1, 2) for w in caps], 2 * P * B)
    print(f"   8 -> 8 copy [16384 x 8192]             {g:9.1f} GB/s  (vec, wg/cu) = {sh}")
    g, sh = best_of(gather, [(nt, w) for nt in (0, 1) for w in (0, 8, 12, 16)], (P + 1) * B)
    print(f"   8 -> 1 XOR gather [16384 x 8192]       {g:9.1f} GB/s  (nt_stores, wg/cu) = {sh}")
    g, sh = best_of(copy_two, [(v, w) for v in (1, 2) for w in caps], 2 * P * B5, s0)
    print(f"   8 -> 8 copy [16384 x 16384], 2 streams {g:9.1f} GB/s  (vec, wg/cu) = {sh}")
    sys.stdout.flush()

    # the bounded ubatch grid's footprint, alone and beside a bf16 GEMM on
    # another stream (one [8192 x 8192] ubatch of the prefill batch, as in
    # tbo_overlap_gemm); the flat grid for comparison
    rows_u = ROWS // 2
    m = rows_u * HIDDEN
    xi, xo = [x[:m] for x in ins], [o[:m] for o in outs]
    gdim = 4096
    ga = torch.randn(gdim, gdim, device=dev, dtype=torch.bfloat16)
    gb = torch.randn(gdim, gdim, device=dev, dtype=torch.bfloat16)
    gc = torch.empty(gdim, gdim, device=dev, dtype=torch.bfloat16)

    def pair(reduce_fn, gemms):
        def step():
            s0.wait_stream(main_s)
            s1.wait_stream(main_s)
            if reduce_fn is not None:
                reduce_fn()
            with torch.cuda.stream(s1):
                for _ in range(gemms):
                    torch.mm(ga, gb, out=gc)
            main_s.wait_stream(s0)
            main_s.wait_stream(s1)
        return timed_settled(torch, main_s, step, 10)

    def red(v):
        return lambda: tar.ar_reduce_ubatch(xi, xo, rows_u, HIDDEN, 1, None, CHUNK_BYTES, v, [s0])

    kb = tar.AR_KERNEL_UBATCH_BOUNDED
    default_b = tar.ar_get_launch_shape(kb)
    t_g1 = pair(None, 1)
    t_flat = pair(red(tar.AR_VARIANT_2STAGE), 0)
    gemms = max(1, round(t_flat / t_g1))
    t_g = pair(None, gemms)
    print(f"== bounded ubatch footprint: one [{rows_u} x {HIDDEN}] ubatch (P=8), alone and beside {gemms} x bf16 "
          f"GEMM {gdim}^3 ({t_g:.4f} ms alone)")
    print("   grid                                alone_ms  with_gemm_ms  overlap  vs_fastest_serial")
    both = pair(red(tar.AR_VARIANT_2STAGE), gemms)
    serial = t_flat + t_g
    print(f"   flat (ubatch default)               {t_flat:8.4f}  {both:12.4f}  {(t_flat + t_g - both) / min(t_flat, t_g):7.2f}"
          f"  {both / serial:17.4f}")
    for block, eighths in ((512, 2), (512, 3), (512, 4), (512, 5), (512, 6), (256, 4), (1024, 4)):
        tar.ar_set_launch_shape(kb, block, 1, 1, 1, eighths)
        v = tar.AR_VARIANT_2STAGE | tar.AR_UBATCH_BOUNDED
        alone = pair(red(v), 0)
        both = pair(red(v), gemms)
        tag = "  <- default" if (block, 1, 1, 1, eighths) == default_b else ""
        print(f"   bounded {block:4d} lanes, {eighths}/8 of the CUs  {alone:8.4f}  {both:12.4f}  "
              f"{(alone + t_g - both) / min(alone, t_g):7.2f}  {both / serial:17.4f}{tag}")
        sys.stdout.flush()
    tar.ar_set_launch_shape(kb, *default_b)
    log("ab: bounded footprint done")
    del ga, gb, gc
    placement_report(tar, torch, dev, main_s, s0, s1, ins, outs, uin, ubo, time_calls)


def ab_small_report(tar, torch, synth, dev, main_s):
    """A/B of the small-message kinds (n <= AR_SMALL_ELEMS) at the decode sizes.

    Each kind -- one-shot, fused two-stage with separate outputs and in
    place, pack, unpack, fused RD, staged RD step -- is timed under every
    (block 64/128/256, plain or non-temporal loads, store policy 0..3) with
    one group per lane and no cap, at 128 KiB, 512 KiB and 2 MiB per rank
    (P = 8), inside a HIP graph of 100 calls replayed 20 times, so the host's
    launch cost does not hide the kernels' differences; three shuffled
    rounds, median.  Score: the geometric mean over the sizes of the time
    against the best shape at that size.  The six best shapes and the
    default are printed per kind."""
    import math
    import random
    import statistics

    side = torch.cuda.Stream()
    sizes = (8, 32, 128)                       # rows of hidden 8192: 128 KiB, 512 KiB, 2 MiB per rank

    def graph_us(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            fn()
            side.synchronize()
            with torch.cuda.graph(g, stream=side):
                for _ in range(100):
                    fn()
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(main_s)
        for _ in range(20):
            g.replay()
        e1.record(main_s)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / 2000

    data = {}
    for T in sizes:
        m = T * HIDDEN
        xs = [x.view(torch.int16) for x in synth.device_rank_buffers("normal", P, m, 3, dev)]
        d = {"xs": xs, "outs": [torch.empty(m, dtype=torch.int16, device=dev) for _ in range(P)],
             "bufs": [x.clone() for x in xs], "x1": torch.empty(m, dtype=torch.int16, device=dev),
             "words": [torch.empty(m // 2, dtype=torch.int64, device=dev) for _ in range(P)],
             "rdo": [torch.empty(m // 2, dtype=torch.int64, device=dev) for _ in range(P)],
             "err": torch.empty(2, dtype=torch.int64, device=dev),
             "mbox": torch.empty(tar.rd_mailbox_words(P, m), dtype=torch.int64, device=dev)}
        for r in range(P):
            tar.ar_pack_fused(xs[r], d["words"][r], 1)
        tar.ar_err_init(d["err"])
        data[T] = d

    def call(kind, d):
        if kind == tar.AR_KERNEL_ONESHOT_SMALL:
            return lambda: tar.ar_reduce_oneshot(d["xs"], d["outs"][0], stream=side)
        if kind == tar.AR_KERNEL_2STAGE_SMALL:
            return lambda: tar.ar_reduce_2stage(d["xs"], d["outs"], stream=side)
        if kind == tar.AR_KERNEL_2STAGE_INPLACE_SMALL:
            return lambda: tar.ar_reduce_2stage(d["bufs"], d["bufs"], stream=side)
        if kind == tar.AR_KERNEL_PACK_SMALL:
            return lambda: tar.ar_pack_fused(d["xs"][0], d["words"][0], 1, stream=side)
        if kind == tar.AR_KERNEL_UNPACK_SMALL:
            return lambda: tar.ar_unpack_fused(d["words"][1], d["x1"], 1, d["err"], stream=side)
        if kind == tar.AR_KERNEL_RD_SMALL:
            return lambda: tar.ar_rd_schedule(d["words"], d["rdo"], 1, d["err"], stream=side)
        return lambda: tar.ar_rd_schedule(d["words"], d["rdo"], 1, d["err"], mailbox=d["mbox"],
                                          flags=tar.AR_RD_STAGED, stream=side)

    kinds = (("ONESHOT_SMALL", tar.AR_KERNEL_ONESHOT_SMALL), ("2STAGE_SMALL", tar.AR_KERNEL_2STAGE_SMALL),
             ("2STAGE_INPLACE_SMALL", tar.AR_KERNEL_2STAGE_INPLACE_SMALL), ("PACK_SMALL", tar.AR_KERNEL_PACK_SMALL),
             ("UNPACK_SMALL", tar.AR_KERNEL_UNPACK_SMALL), ("RD_SMALL", tar.AR_KERNEL_RD_SMALL),
             ("RDSTEP_SMALL", tar.AR_KERNEL_RDSTEP_SMALL))
    cands = [(b, 1, l, st, 0) for b in (64, 128, 256) for l in (0, 1) for st in (0, 1, 2, 3)]
    props = torch.cuda.get_device_properties(dev)
    print("# A/B of the small-message kinds at the decode sizes: P=8, [T x 8192] per rank, T = 8 / 32 / 128")
    print("# command: python bench.py --ab-small   (per-call time inside HIP graphs of 100 calls, "
          "3 shuffled rounds, median)")
    print(f"# device: {props.name}, {props.multi_processor_count} CUs")
    print("# score: geometric mean over the sizes of time / best time at that size (1.000 = best everywhere)")
    rng = random.Random(17)
    for name, kind in kinds:
        default = tar.ar_get_launch_shape(kind)
        cs = cands + ([default] if default not in cands else [])
        t = {(c, T): [] for c in cs for T in sizes}
        for _ in range(3):
            order = list(t)
            rng.shuffle(order)
            for c, T in order:
                tar.ar_set_launch_shape(kind, *c)
                t[(c, T)].append(graph_us(call(kind, data[T])))
        tar.ar_set_launch_shape(kind, *default)
        med = {k: statistics.median(v) for k, v in t.items()}
        best = {T: min(med[(c, T)] for c in cs) for T in sizes}
        score = {c: math.exp(sum(math.log(med[(c, T)] / best[T]) for T in sizes) / len(sizes)) for c in cs}
        ranked = sorted(cs, key=lambda c: score[c])
        print(f"== {name}: default {default}")
        print("   block vec ntl stores wg/cu   score    128KiB     512KiB    2048KiB")
        for c in ranked[:6] + ([default] if default not in ranked[:6] else []):
            tag = "  <- default" if c == default else ""
            print(f"   {c[0]:5d} {c[1]:3d} {c[2]:3d} {c[3]:6d} {c[4]:5d}  {score[c]:6.3f}  "
                  + "  ".join(f"{med[(c, T)]:7.2f}us" for T in sizes) + tag)
        sys.stdout.flush()
        log(f"ab-small: {name} done")


def placement_report(tar, torch, dev, main_s, s0, s1, ins, outs, uin, ubo, time_calls):
    """The 8 -> 8 rate against where the 16 buffers sit relative to one another.

    The P simulated ranks' buffers share one GPU's HBM (with P real ranks each
    rank reads its own), and the DRAM channel and bank an address maps to
    depends on its higher address bits: 16 streams whose bases differ only in
    some of those bits contend for the same banks at the same offset.  The
    fused two-stage runs on 16 buffers of 256 MiB carved from one pooled
    allocation at stride S, inputs first then outputs, or alternating; the
    two-ubatch reduce runs on 16 buffers of 512 MiB at stride 512 MiB + skew.
    The bench's own separately allocated buffers are the first row of each
    table.  Pool contents are arbitrary finite bf16 patterns; the rate does
    not depend on the values."""
    import random
    import statistics

    n = ROWS * HIDDEN
    n5 = UB_ROWS * UB_HIDDEN
    MiB = 1 << 20
    strides = (256, 256.25, 258, 260, 264, 288, 384, 512)
    skews = (0, 0.25, 2, 8, 128)
    span = max(16 * max(strides) * MiB // 2, 16 * (512 + max(skews)) * MiB // 2)
    pool = torch.empty(int(span) + n5, dtype=torch.int16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    pool.random_(-16000, 16000, generator=g)

    def carve(stride_mib, count, elems, alternating):
        e = int(stride_mib * MiB) // 2
        b = [pool[k * e:k * e + elems] for k in range(2 * count)]
        return (b[0::2], b[1::2]) if alternating else (b[:count], b[count:])

    # two-stream calls by the timing protocol, timed on stream A (s0)
    u_start, u_bend = torch.cuda.Event(), torch.cuda.Event()

    def ubatch(i, o, streams):
        a, b = streams

        def fn():
            if b is not a:
                u_start.record(a)
                b.wait_event(u_start)
            tar.ar_reduce_ubatch(i, o, UB_ROWS, UB_HIDDEN, 2, None, CHUNK_BYTES, tar.AR_VARIANT_2STAGE, streams)
            if b is not a:
                u_bend.record(b)
                a.wait_event(u_bend)
        return fn

    c4 = {"separate allocations (bench)": lambda: tar.ar_reduce_2stage(ins, outs)}
    for S in strides:
        for alt in (False, True):
            i, o = carve(S, P, n, alt)
            c4[f"stride {S:g} MiB, {'alternating' if alt else 'inputs then outputs'}"] = (
                lambda i=i, o=o: tar.ar_reduce_2stage(i, o))
    c5 = {}
    for mode, streams in (("two streams", [s0, s1]), ("one stream", [s0, s0])):
        c5[f"separate allocations (bench), {mode}"] = ubatch(uin, ubo, streams)
        for sk in skews:
            i, o = carve(512 + sk, P, n5, False)
            c5[f"stride 512 MiB + {sk:g} MiB, {mode}"] = ubatch(i, o, streams)
    rng = random.Random(13)
    rounds = 3
    print("== buffer placement: the 8 -> 8 rate against the buffers' relative addresses "
          f"({rounds} shuffled rounds, median)")
    for title, cases, cred, tst in (("fused two-stage, P=8, 16 buffers of 256 MiB", c4, 2 * P * 2 * n, None),
                                    ("two-ubatch reduce, P=8, 16 buffers of 512 MiB", c5, 2 * P * 2 * n5, s0)):
        times = {k: [] for k in cases}
        for _ in range(rounds):
            order = list(cases)
            rng.shuffle(order)
            for k in order:
                times[k].append(time_calls(cases[k], tst))
        print(f"   {title}")
        print("   placement                                              ms      GB/s  frac-of-8TB/s")
        for k in cases:
            ms = statistics.median(times[k])
            gbps = cred / (ms * 1e-3) / 1e9
            print(f"   {k:50s} {ms:9.4f} {gbps:9.1f}  {gbps / PEAK_HBM_GBPS:13.4f}")
        sys.stdout.flush()
    del pool
    torch.cuda.empty_cache()
    log("ab: placement done")


def overlap(tar, blib, torch, dev, main_s, ins, outs, s0, s1):
    """Two-stream overlap on one GPU.

    tbo: the two-stage reduce of one 8192-row ubatch on the comm stream s0,
    beside an ALU-bound stand-in for the partner ubatch's compute on s1 sized
    to take about as long; overlap = (t_reduce + t_compute - t_both) /
    min(t_reduce, t_compute).
    chunk_pipeline: the same reduce with per-chunk completion flags, and a
    consumer on s1 that takes each 1 MiB chunk of one output as soon as its
    flag is set, compared with running the two one after the other.  Two
    consumers: a plain copy (HBM-bound like the reduce, so the two share the
    bandwidth and overlap cannot shorten the makespan), and the copy plus
    FMA work per word sized to take about as long as the reduce (the case
    per-chunk flags are for: the consumer's compute hides the reduce)."""
    rows = ROWS // 2
    m = rows * HIDDEN
    xi = [x[:m] for x in ins]
    xo = [o[:m] for o in outs]
    alu_grid = 512
    alu_out = torch.empty(alu_grid * 256, dtype=torch.float32, device=dev)
    dst = torch.empty(m, dtype=torch.int16, device=dev)
    nchunks = tar.ubatch_chunk_count(rows, HIDDEN, 1, None, CHUNK_BYTES)
    done = torch.zeros(nchunks, dtype=torch.int32, device=dev)
    tiles = torch.zeros(nchunks, dtype=torch.int32, device=dev)
    timeouts = torch.zeros(1, dtype=torch.int32, device=dev)
    epoch = [0]

    def reduce(flags=False, bounded=False):
        if flags:
            epoch[0] += 1
            tar.ar_reduce_ubatch_flags(xi, xo, rows, HIDDEN, done, tiles, epoch[0], 1, None, CHUNK_BYTES,
                                       tar.AR_VARIANT_2STAGE, [s0])
        else:
            v = tar.AR_VARIANT_2STAGE | (tar.AR_UBATCH_BOUNDED if bounded else 0)
            tar.ar_reduce_ubatch(xi, xo, rows, HIDDEN, 1, None, CHUNK_BYTES, v, [s0])

    def compute(iters):
        if blib.arb_alu(alu_out.data_ptr(), iters, alu_grid, s1.cuda_stream) != 0:
            raise RuntimeError("arb_alu failed")

    cons_grid = 2 * torch.cuda.get_device_properties(dev).multi_processor_count   # most a waiting consumer may take
    sink = torch.zeros(cons_grid * 256, dtype=torch.float32, device=dev)

    def consume(work=0):
        if blib.arb_consume_chunks(done.data_ptr(), epoch[0], xo[0].data_ptr(), dst.data_ptr(), m,
                                   CHUNK_BYTES // 2, 0, 1 << 24, timeouts.data_ptr(), work,
                                   sink.data_ptr() if work else None, cons_grid, s1.cuda_stream) != 0:
            raise RuntimeError("arb_consume_chunks failed")

    def timed(fn, reps=10):
        def step():
            s0.wait_stream(main_s)
            s1.wait_stream(main_s)
            fn()
            main_s.wait_stream(s0)
            main_s.wait_stream(s1)
        return timed_settled(torch, main_s, step, reps)

    t_r = timed(lambda: reduce())
    iters = 4096
    t_c = timed(lambda: compute(iters))
    iters = max(64, int(iters * t_r / t_c))
    t_c = timed(lambda: compute(iters))
    t_both = timed(lambda: (reduce(), compute(iters)))
    ov = (t_r + t_c - t_both) / min(t_r, t_c)
    # the partner ubatch's compute as a real bf16 GEMM (MFMA-bound; plain 2-D
    # product with contiguous operands) sized to take about as long as the reduce
    gdim = 4096
    ga = torch.randn(gdim, gdim, device=dev, dtype=torch.bfloat16)
    gb = torch.randn(gdim, gdim, device=dev, dtype=torch.bfloat16)

    gc = torch.empty(gdim, gdim, device=dev, dtype=torch.bfloat16)

    def gemm(reps):
        with torch.cuda.stream(s1):
            for _ in range(reps):
                torch.mm(ga, gb, out=gc)

    t_g = timed(lambda: gemm(1))
    gemm_flop = 2 * gdim ** 3
    reps_g = max(1, round(t_r / t_g))
    t_g = timed(lambda: gemm(reps_g))
    t_gboth = timed(lambda: (reduce(), gemm(reps_g)))
    ov_g = (t_r + t_g - t_gboth) / min(t_r, t_g)
    log(f"overlap with a bf16 GEMM: reduce {t_r:.3f} ms, {reps_g} x GEMM {gdim}^3 {t_g:.3f} ms, "
        f"both {t_gboth:.3f} ms -> {ov_g:.2f}")
    # the same with the reduce on its bounded-footprint grid (a persistent
    # grid on part of the CUs), which leaves the rest of the device to the
    # GEMM: slower alone, but the pair finishes sooner than either order of
    # the fastest reduce and the GEMM one after the other
    t_rb = timed(lambda: reduce(bounded=True))
    t_gbb = timed(lambda: (reduce(bounded=True), gemm(reps_g)))
    ov_b = (t_rb + t_g - t_gbb) / min(t_rb, t_g)
    log(f"overlap with a bf16 GEMM, bounded reduce: reduce {t_rb:.3f} ms, both {t_gbb:.3f} ms -> {ov_b:.2f}; "
        f"serial with the fastest reduce {t_r + t_g:.3f} ms")
    del ga, gb, gc
    t_rf = timed(lambda: reduce(True))
    t_cons = timed(lambda: consume())           # flags already set: the consumer alone
    t_pipe = timed(lambda: (reduce(True), consume()))
    work = 64
    t_w = timed(lambda: consume(work))
    for _ in range(2):                          # the copy part does not scale with work
        work = max(1, int(work * t_rf / t_w))
        t_w = timed(lambda: consume(work))
    t_wpipe = timed(lambda: (reduce(True), consume(work)))
    torch.cuda.synchronize()
    if int(timeouts.item()) != 0:
        raise RuntimeError("chunk consumer timed out")
    ov_w = (t_rf + t_w - t_wpipe) / min(t_rf, t_w)
    log(f"overlap: reduce {t_r:.3f} ms, compute {t_c:.3f} ms, both {t_both:.3f} ms -> {ov:.2f}; "
        f"chunk pipeline: copy consumer {t_pipe:.3f} ms vs serial {t_rf + t_cons:.3f} ms; "
        f"compute consumer {t_wpipe:.3f} ms vs serial {t_rf + t_w:.3f} ms -> {ov_w:.2f}")
    return {"tbo_overlap": {"reduce_ms": round(t_r, 4), "compute_ms": round(t_c, 4),
                            "both_ms": round(t_both, 4), "overlap_fraction": round(ov, 3),
                            "reduce": "two-stage, one ubatch of [8192 x 8192] x 8 ranks, 1 MiB chunks",
                            "compute": f"ALU stand-in, {alu_grid} x 256 lanes, {iters} FMA rounds"},
            "tbo_overlap_gemm": {"gemm_ms": round(t_g, 4),
                                 "gemm": f"{reps_g} x bf16 [{gdim} x {gdim}] x [{gdim} x {gdim}] (torch.mm)",
                                 "gemm_TFLOPs": round(reps_g * gemm_flop / (t_g * 1e-3) / 1e12, 1),
                                 "flat_grid": {"reduce_ms": round(t_r, 4), "both_ms": round(t_gboth, 4),
                                               "overlap_fraction": round(ov_g, 3)},
                                 "bounded_grid": {"reduce_ms": round(t_rb, 4), "both_ms": round(t_gbb, 4),
                                                  "overlap_fraction": round(ov_b, 3),
                                                  "shape": list(tar.ar_get_launch_shape(tar.AR_KERNEL_UBATCH_BOUNDED))},
                                 "serial_fastest_ms": round(t_r + t_g, 4),
                                 "bounded_makespan_over_serial": round(t_gbb / (t_r + t_g), 4)},
            "chunk_pipeline": {"flagged_reduce_ms": round(t_rf, 4), "chunks": nchunks,
                               "copy_consumer": {"alone_ms": round(t_cons, 4),
                                                 "serial_ms": round(t_rf + t_cons, 4),
                                                 "pipelined_ms": round(t_pipe, 4)},
                               "compute_consumer": {"fma_rounds_per_16B": work, "alone_ms": round(t_w, 4),
                                                    "serial_ms": round(t_rf + t_w, 4),
                                                    "pipelined_ms": round(t_wpipe, 4),
                                                    "overlap_fraction": round(ov_w, 3)}}}


def timed_settled(torch, stream, fn, reps, settle_s=0.03):
    """Mean ms per call over `reps` back-to-back calls of fn, timed with
    events on `stream` (fn launches there), after at least `settle_s` seconds
    of the same calls.  After an idle gap the GPU dips below its working
    clock for about 20 ms of load; the memory-bound kernels do not feel it,
    but the fp8 quantise (the most arithmetic per byte here) ran up to 25%
    slower inside the dip."""
    settle = time.perf_counter() + settle_s
    while time.perf_counter() < settle:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def wait_receive(tar, blib, torch, dev, main_s, ins, outs, s0, s1):
    """The waiting unpack (ar_unpack_fused_wait).

    prefill: all 8 rank payloads of the [16384 x 8192] batch already carry
    the expected sequence number; the waiting unpack against the plain one
    (3 B per element each: payload read, bf16 written).
    decode_handoff: one rank's [128 x 8192] message through the native loop
    arb_handoff_us: the producer packs it on s0 with a new sequence number
    each time and the consumer, queued after it on s1 with no dependency on
    it, polls until its words carry that number.  Median time from before the
    pack to after the unpack, against the same pack and a plain unpack one
    after the other on one stream; every handoff must complete with no stale
    word."""
    def timed(fn, reps):
        return timed_settled(torch, main_s, fn, reps)

    n = ROWS * HIDDEN
    err = torch.empty(2, dtype=torch.int64, device=dev)
    tar.ar_err_init(err, stream=main_s)
    words = [torch.empty(n // 2, dtype=torch.int64, device=dev) for _ in range(P)]
    for r in range(P):
        tar.ar_pack_fused(ins[r], words[r], 7)
    b = P * 3 * 2 * n
    t_plain = timed(lambda: [tar.ar_unpack_fused(words[r], outs[r], 7, err) for r in range(P)], 5)
    t_wait = timed(lambda: [tar.ar_unpack_fused_wait(words[r], outs[r], 7, err) for r in range(P)], 5)
    del words
    torch.cuda.empty_cache()
    m = 128 * HIDDEN
    w1 = torch.empty(m // 2, dtype=torch.int64, device=dev)
    x1 = torch.empty(m, dtype=torch.int16, device=dev)
    x0 = ins[0][:m]
    torch.cuda.synchronize()

    def handoff(serial, seq0):
        us = blib.arb_handoff_us(x0.data_ptr(), w1.data_ptr(), x1.data_ptr(), m, seq0, err.data_ptr(), 300,
                                 serial, (main_s if serial else s0).cuda_stream, s1.cuda_stream)
        if us < 0:
            raise RuntimeError(f"arb_handoff_us failed: {us}")
        return us

    t_hand = handoff(0, 1000)
    t_ser = handoff(1, 5000)
    torch.cuda.synchronize()
    stale = int(err[0].item())
    if stale:
        raise RuntimeError(f"waiting unpack left {stale} stale payload words")
    if not torch.equal(x1, x0):
        raise RuntimeError("waiting unpack: data differs from the packed input")
    g = lambda t: round(b / (t * 1e-3) / 1e9, 1)
    log(f"waiting unpack: prefill {t_wait:.3f} ms vs plain {t_plain:.3f} ms; decode handoff {t_hand:.2f} us "
        f"(pack then plain unpack on one stream {t_ser:.2f} us)")
    return {"wait_receive": {
        "prefill": {"wait_ms": round(t_wait, 4), "wait_GBps": g(t_wait), "plain_ms": round(t_plain, 4),
                    "plain_GBps": g(t_plain), "unpacks": P},
        "decode_handoff_128x8192": {"waiting_us": round(t_hand, 2), "serial_pack_unpack_us": round(t_ser, 2),
                                    "measure": "median, event before the pack to event after the unpack"}}}


def fp8(tar, torch, dev, main_s, ins, outs):
    """fp8-quantised contributions at the prefill shape (P = 8, [16384 x
    8192] per rank) and at the decode sizes: quantise all P buffers (one
    launch), then reduce into one output or into all P.  Algorithmic bytes:
    quantise P (2n + n + n/32), reduce P (n + n/32) + 2n per output."""
    def timed(fn, reps):
        return timed_settled(torch, main_s, fn, reps)

    n = ROWS * HIDDEN
    nb = tar.fp8_scale_count(n)
    codes = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(P)]
    scales = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(P)]
    b_q = P * (3 * n + nb)
    b_r1 = P * (n + nb) + 2 * n
    b_rp = P * (n + nb) + P * 2 * n
    t_q = timed(lambda: tar.ar_quantize_fp8(ins, codes, scales), 20)
    t_r1 = timed(lambda: tar.ar_reduce_fp8(codes, scales, outs[:1]), 20)
    t_rp = timed(lambda: tar.ar_reduce_fp8(codes, scales, outs), 20)
    g = lambda b, t: round(b / (t * 1e-3) / 1e9, 1)
    res = {"quantize_x8": {"ms": round(t_q, 4), "GBps": g(b_q, t_q), "frac_of_peak": round(g(b_q, t_q) / PEAK_HBM_GBPS, 4)},
           "reduce_one_output": {"ms": round(t_r1, 4), "GBps": g(b_r1, t_r1),
                                 "frac_of_peak": round(g(b_r1, t_r1) / PEAK_HBM_GBPS, 4)},
           "reduce_all_outputs": {"ms": round(t_rp, 4), "GBps": g(b_rp, t_rp),
                                  "frac_of_peak": round(g(b_rp, t_rp) / PEAK_HBM_GBPS, 4)}}
    log(f"fp8 prefill: quantise {t_q:.3f} ms ({g(b_q, t_q):.0f} GB/s), reduce->1 {t_r1:.3f} ms "
        f"({g(b_r1, t_r1):.0f} GB/s), reduce->{P} {t_rp:.3f} ms ({g(b_rp, t_rp):.0f} GB/s)")
    del codes, scales
    # decode sizes: 100 calls captured in one HIP graph, replayed (per-call
    # time without the host's launch cost, as in latency_hip_graph)
    side = torch.cuda.Stream()
    side.wait_stream(main_s)

    def graph_us(fn):
        with torch.cuda.stream(side):
            fn(side)
            side.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=side):
                for _ in range(100):
                    fn(side)
        torch.cuda.synchronize()
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main_s)
        for _ in range(20):
            gr.replay()
        e1.record(main_s)
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / 2000, 2)

    lat = {}
    for T in (8, 32, 128):
        m = T * HIDDEN
        xi = [x[:m] for x in ins]
        xo = [o[:m] for o in outs]
        cs = [torch.empty(m, dtype=torch.uint8, device=dev) for _ in range(P)]
        ss = [torch.empty(tar.fp8_scale_count(m), dtype=torch.uint8, device=dev) for _ in range(P)]
        lat[f"{2 * m // 1024}KiB"] = {
            "quantize_x8": graph_us(lambda st: tar.ar_quantize_fp8(xi, cs, ss, stream=st)),
            "reduce_one": graph_us(lambda st: tar.ar_reduce_fp8(cs, ss, xo[:1], stream=st)),
            "reduce_all": graph_us(lambda st: tar.ar_reduce_fp8(cs, ss, xo, stream=st))}
    res["decode_us_per_call_hip_graph"] = lat
    log("fp8 decode sizes timed")
    return {"fp8": res}


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, np):
    """The oracle (single-threaded C, as it stands) on a bounded sample of the
    same step: the first `rows_s` rows of both batches -- [rows_s x 8192] for
    the one-shot, two-stage, pack, RD and unpack rows, [rows_s x 16384] split
    into two ubatches for the ubatch row."""
    import oracle
    from tensor_all_reduce_amd import synth

    def gen(rows_s):
        return ([synth.normal(rows_s * HIDDEN, 4, 0, p) for p in range(P)],
                [synth.logmag(rows_s * UB_HIDDEN, 5, 0, p) for p in range(P)])

    def step(rows_s, data=None, barrier=None):
        m, m5 = rows_s * HIDDEN, rows_s * UB_HIDDEN
        xs, x5 = gen(rows_s) if data is None else data
        if barrier is not None:
            barrier.wait()
        t0 = time.perf_counter()
        oracle.reduce_seq(xs)
        oracle.reduce_2stage(xs)
        ws = [oracle.pack(x, 1) for x in xs]
        rw, _ = oracle.rd(ws, 1)
        for w in rw:
            oracle.unpack(w, 4)
        oracle.reduce_ubatch(x5, rows_s, UB_HIDDEN, 2, None, CHUNK_BYTES // 2, oracle.TWOSTAGE)
        t1 = time.perf_counter()
        b, b5 = 2 * m, 2 * m5
        cred = (P + 1) * b + 2 * P * b + 3 * P * b + 4 * P * b + 3 * P * b + 2 * P * b5
        if barrier is not None:
            return t0, t1, cred
        return t1 - t0, cred

    # size the sample from a 128-row run, then once more from the sample
    # itself if that came out under half the target: the cost per row grows
    # once the rows no longer fit the host's caches, and a short run is noisy
    dt, _ = step(128)
    rows_s = int(min(ROWS, max(128, 128 * args.cpu_seconds / max(dt, 1e-3))))
    rows_s -= rows_s % 2
    log(f"cpu oracle: calibration 128 rows took {dt:.2f} s; timing {rows_s} rows")
    dt, cred = step(rows_s)
    if dt < 0.5 * args.cpu_seconds and rows_s < ROWS:
        rows_s = int(min(ROWS, rows_s * args.cpu_seconds / max(dt, 1e-3)))
        rows_s -= rows_s % 2
        log(f"cpu oracle: {dt:.1f} s, under half the target; timing {rows_s} rows")
        dt, cred = step(rows_s)
    gbps = cred / dt / 1e9
    res = {"value": round(gbps, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"one full step (all six rows) of the oracle on the first {rows_s} of 16384 rows of both "
                     f"batches (P=8; hidden 8192 N(0,1), and hidden 16384 log-uniform for the ubatch row); "
                     f"{dt:.1f} s on one host core; credited bytes as the GPU step",
           "seconds": round(dt, 2), "cpu_model": cpu_model()}
    if args.no_cpu_all_cores:
        return res
    # the same oracle on every host core this process may use: one thread
    # per core, each running the unchanged oracle on its own rows (the C
    # calls release the interpreter lock)
    import concurrent.futures as cf
    import threading
    cores = max(1, len(os.sched_getaffinity(0)))
    rows_t = max(2, min(rows_s, ROWS // cores))
    rows_t -= rows_t % 2
    data = gen(rows_t)                     # every thread reduces the same values
    barrier = threading.Barrier(cores)
    with cf.ThreadPoolExecutor(cores) as ex:
        parts = list(ex.map(lambda _: step(rows_t, data, barrier), range(cores)))
    wall = max(t1 for _, t1, _ in parts) - min(t0 for t0, _, _ in parts)
    cred_all = sum(c for _, _, c in parts)
    res["all_cores"] = {"value": round(cred_all / wall / 1e9, 3), "unit": "GB/s", "cores": cores,
                        "seconds": round(wall, 2),
                        "sample": f"{cores} threads, each one full oracle step on {rows_t} rows of its own"}
    log(f"cpu oracle on {cores} cores: {res['all_cores']['value']} GB/s")
    return res


if __name__ == "__main__":
    sys.exit(main())
