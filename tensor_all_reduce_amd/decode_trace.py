"""Profiling target for decode-size calls: a fixed sequence of library calls
at the decode message sizes, so that a rocprofv3 kernel trace gives the
kernel-only duration of each (the third latency figure beside the stream
time per call and the wall time per call that bench.py reports).

Phases run one after another; each is `reps` calls of one entry point at
one size.  The plan (phase name, library dispatches per call, calls, bytes
credited per call) is written as JSON so that `profsum decode` can label
the trace's library dispatches by their position.

Usage:
  python -m tensor_all_reduce_amd.decode_trace --plan out/decode_plan.json --reps 200
"""
from __future__ import annotations

import argparse
import json
import sys

HIDDEN = 8192


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--plan", required=True, help="where to write the phase plan (JSON)")
    ap.add_argument("--reps", type=int, default=200)
    a = ap.parse_args(argv)

    import torch

    import tensor_all_reduce_amd as tar
    from tensor_all_reduce_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    tar.lib()
    dev = torch.device("cuda:0")
    P = 8
    nmax = 128 * HIDDEN
    ins = [t.view(torch.int16) for t in synth.device_rank_buffers("normal", P, nmax, 3, dev)]
    outs = [torch.empty(nmax, dtype=torch.int16, device=dev) for _ in range(P)]
    scratch = torch.empty(nmax, dtype=torch.int16, device=dev)
    win = [torch.empty(nmax // 2, dtype=torch.int64, device=dev) for _ in range(P)]
    wout = [torch.empty(nmax // 2, dtype=torch.int64, device=dev) for _ in range(P)]
    mbox = torch.empty(tar.rd_mailbox_words(P, nmax), dtype=torch.int64, device=dev)
    err = torch.empty(2, dtype=torch.int64, device=dev)
    s = torch.cuda.current_stream()
    plan = []

    def phase(name, per_call, credited, fn):
        for _ in range(a.reps):
            fn()
        torch.cuda.synchronize()
        plan.append({"phase": name, "dispatches_per_call": per_call, "calls": a.reps,
                     "credited_bytes_per_call": credited})
        print(f"[decode_trace] {name}: {a.reps} calls", flush=True)

    # P = 2, one token: [1 x 8192]
    m = HIDDEN
    phase("oneshot P=2 16KiB", 1, 3 * 2 * m,
          lambda: tar.ar_reduce_oneshot([x[:m] for x in ins[:2]], outs[0][:m], stream=s))
    for T in (8, 32, 128):
        m = T * HIDDEN
        xi = [x[:m] for x in ins]
        xo = [o[:m] for o in outs]
        kib = 2 * m // 1024
        phase(f"oneshot P=8 {kib}KiB", 1, (P + 1) * 2 * m,
              lambda: tar.ar_reduce_oneshot(xi, xo[0], stream=s))
        phase(f"2stage_fused P=8 {kib}KiB", 1, 2 * P * 2 * m,
              lambda: tar.ar_reduce_2stage(xi, xo, stream=s))
        phase(f"2stage_staged P=8 {kib}KiB", 2, 2 * P * 2 * m,
              lambda: tar.ar_reduce_2stage(xi, xo, scratch=scratch[:m], stream=s))
    # fused payloads at [128 x 8192]
    m = nmax
    xi, xo = ins, outs
    for p in range(P):
        tar.ar_pack_fused(xi[p], win[p], 1, stream=s)
    tar.ar_err_init(err, stream=s)
    torch.cuda.synchronize()
    plan.append({"phase": "setup", "dispatches_per_call": P + 1, "calls": 1, "credited_bytes_per_call": 0})
    phase("pack 2MiB", 1, 3 * 2 * m, lambda: tar.ar_pack_fused(xi[0], win[0], 1, stream=s))
    phase("rd_fused_R1 P=8 2MiB", 1, 4 * P * 2 * m, lambda: tar.ar_rd_schedule(win, wout, 1, err, stream=s))
    phase("rd_fused_R2 P=8 2MiB", 1, 4 * P * 2 * m,
          lambda: tar.ar_rd_schedule(win, wout, 1, err, flags=tar.AR_RD_FP32_CARRY, stream=s))
    phase("rd_staged_R1 P=8 2MiB", 3, 4 * P * 2 * m,
          lambda: tar.ar_rd_schedule(win, wout, 1, err, mailbox=mbox, flags=tar.AR_RD_STAGED, stream=s))
    phase("unpack 2MiB", 1, 3 * 2 * m, lambda: tar.ar_unpack_fused(wout[0], xo[0], 4, err, stream=s))
    torch.cuda.synchronize()
    e = err.cpu().tolist()
    if e[0] != 0:
        raise SystemExit(f"decode trace saw {e[0]} bad sequence numbers")
    with open(a.plan, "w") as f:
        json.dump(plan, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
