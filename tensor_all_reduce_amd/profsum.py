"""Summarise rocprofv3 CSV output of bench.py into short text files.

  stats    kernel durations from a --kernel-trace --stats run: per hot-path
           row, the rocprofv3 average over all dispatches and the average
           over the timed steps only (warmup steps dropped), next to the
           rocprofv3 kernel_stats line.
  pmc      any counters from one or more --pmc runs of the bench step:
           per row, the mean per dispatch of every counter collected, and
           derived figures (bytes per VMEM instruction, L2 hit rate).
  kstats   the rocprofv3 --stats per-kernel table (calls, average, min,
           max) of any run, and per kernel the mean FETCH_SIZE / WRITE_SIZE
           of a matching --pmc run when one is given.
  decode   kernel-only durations of the decode-size calls that
           decode_trace.py issues, labelled by the plan it writes.
  traffic  HBM bytes per launch from two --pmc runs (FETCH_SIZE, then
           WRITE_SIZE; KiB per dispatch), each scaled by what the same
           counter reads for the plain 1 GiB copies that bench.py
           --copy-calib appends (known bytes / counted bytes).

Dispatches are labelled by position: every bench step launches the same
sequence of library kernels (STEP below), so the n-th library dispatch of a
step is that row's kernel whatever its template arguments.

Usage:
  python -m tensor_all_reduce_amd.profsum stats DIR --warmup W --command "..."
  python -m tensor_all_reduce_amd.profsum decode DIR PLAN.json --command "..."
  python -m tensor_all_reduce_amd.profsum pmc DIR [DIR ...] --command "..." [--command "..."]
  python -m tensor_all_reduce_amd.profsum traffic FETCH_DIR WRITE_DIR --calib-bytes B \
      --command-fetch "..." --command-write "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 8
# library kernels launched by one bench step, in launch order
STEP = (["oneshot", "2stage"] + ["pack"] * P + ["err_init", "rd"] + ["unpack"] * P + ["ubatch"] * 2)
ROWS = ["oneshot", "2stage", "pack", "rd", "unpack", "ubatch"]
LAUNCHES = {"oneshot": 1, "2stage": 1, "pack": P, "rd": 1, "unpack": P, "ubatch": 2}
PREFIX = {"oneshot": "k_reduce", "2stage": "k_reduce", "pack": "k_pack", "err_init": "k_err_init",
          "rd": "k_rd_fused", "unpack": "k_unpack", "ubatch": "k_reduce"}
# algorithmic bytes per launch: [16384 x 8192] bf16 per rank buffer, and
# [16384 x 16384] for the ubatch row (each of its two launches reduces one
# 8192-row ubatch of every rank: P * B5 / 2 read, P * B5 / 2 written)
B = 2 * 16384 * 8192
B5 = 2 * 16384 * 16384
ALGO = {"oneshot": (P + 1) * B, "2stage": 2 * P * B, "pack": 3 * B, "rd": 4 * P * B,
        "unpack": 3 * B, "ubatch": P * B5}
SOURCES = ["tensor_all_reduce_amd/csrc/ar_device.hpp", "tensor_all_reduce_amd/csrc/ar_reduce.hip",
           "tensor_all_reduce_amd/csrc/ar_fused.hip", "tensor_all_reduce_amd/csrc/ar_api.hip"]


def sources_sha256() -> str:
    h = hashlib.sha256()
    for p in SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def one(pattern: str) -> str:
    hits = glob.glob(pattern)
    if len(hits) != 1:
        raise SystemExit(f"expected one file for {pattern}, found {hits}")
    return hits[0]


def label(rows, name_key, order_key):
    """Library dispatches in launch order, each tagged with its row."""
    lib = [r for r in rows if "ar::k_" in r[name_key]]
    lib.sort(key=lambda r: int(r[order_key]))
    steps = len(lib) // len(STEP)
    out = []
    for s in range(steps):
        for i, row in enumerate(STEP):
            r = lib[s * len(STEP) + i]
            if PREFIX[row] not in r[name_key]:
                raise SystemExit(f"dispatch {s}/{i}: expected {PREFIX[row]}, found {r[name_key][:60]}")
            out.append((s, row, r))
    return out, steps


def cmd_stats(a):
    trace = one(os.path.join(a.dir, "*kernel_trace.csv"))
    stats = one(os.path.join(a.dir, "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(trace)))
    lab, steps = label(rows, "Kernel_Name", "Dispatch_Id")
    dur = {r: [] for r in ROWS}
    dur_all = {r: [] for r in ROWS}
    span = {}                         # (step) -> [start, end] of the two concurrent ubatch launches
    for s, row, r in lab:
        if row not in dur:
            continue
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        d = (t1 - t0) * 1e-6
        dur_all[row].append(d)
        if s >= a.warmup:
            dur[row].append(d)
            if row == "ubatch":
                lo, hi = span.get(s, (t0, t1))
                span[s] = (min(lo, t0), max(hi, t1))
    print(f"# rocprofv3 kernel trace of the bench step: P=8, bf16 [16384 x 8192] per rank "
          f"([16384 x 16384] for the ubatch row)")
    print(f"# command: {a.command}")
    print(f"# {steps} steps traced, first {a.warmup} are warmup; durations in ms per dispatch")
    print(f"# row      launches/step  mean(timed)  median(timed)  mean(all)  algorithmic GB/s per launch")
    for row in ROWS:
        m = statistics.mean(dur[row])
        gbps = ALGO[row] / (m * 1e-3) / 1e9
        print(f"{row:9s} {LAUNCHES[row]:3d}  {m:10.4f}  {statistics.median(dur[row]):10.4f}  "
              f"{statistics.mean(dur_all[row]):10.4f}  {gbps:8.1f}")
    mk = statistics.mean([(hi - lo) * 1e-6 for lo, hi in span.values()])
    print(f"# ubatch: the two launches run concurrently on two streams; mean makespan per step "
          f"{mk:.4f} ms = {2 * ALGO['ubatch'] / (mk * 1e-3) / 1e9:.1f} GB/s for both ubatches")
    print("#")
    print("# rocprofv3 --stats kernel_stats.csv (library kernels), all dispatches of the run:")
    for r in csv.DictReader(open(stats)):
        if "ar::k_" in r["Name"] or "k_copy" in r["Name"]:
            name = r["Name"].split("(")[0].replace("void ", "")
            print(f"#   {name:48s} calls {int(r['Calls']):4d}  avg {float(r['AverageNs']) * 1e-6:.4f} ms  "
                  f"min {float(r['MinNs']) * 1e-6:.4f}  max {float(r['MaxNs']) * 1e-6:.4f}")


def cmd_decode(a):
    import json
    trace = one(os.path.join(a.dir, "*kernel_trace.csv"))
    rows = [r for r in csv.DictReader(open(trace)) if "ar::k_" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    plan = json.load(open(a.plan))
    need = sum(p["dispatches_per_call"] * p["calls"] for p in plan)
    if need != len(rows):
        raise SystemExit(f"plan covers {need} library dispatches, trace has {len(rows)}")
    print("# rocprofv3 kernel trace of decode-size calls (kernel-only time per call, launch excluded)")
    print(f"# command: {a.command}")
    print("# per call: sum of its dispatches' durations; first 10% of calls of each phase dropped")
    print(f"# {'phase':28s} {'calls':>5s} {'mean_us':>8s} {'p50_us':>8s} {'p10_us':>8s} {'p90_us':>8s} "
          f"{'GB/s(p50)':>9s}  kernels")
    i = 0
    for p in plan:
        k, c = p["dispatches_per_call"], p["calls"]
        calls = []
        names = []
        for j in range(c):
            ds = rows[i + j * k: i + (j + 1) * k]
            calls.append(sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in ds) * 1e-3)
            if j == 0:
                names = [r["Kernel_Name"].split("(")[0].replace("void ", "") for r in ds]
        i += k * c
        if p["phase"] == "setup":
            continue
        t = sorted(calls[c // 10:])
        p50 = statistics.median(t)
        gb = p["credited_bytes_per_call"] / (p50 * 1e-6) / 1e9 if p["credited_bytes_per_call"] else 0.0
        uniq = sorted(set(names), key=names.index)
        print(f"{p['phase']:30s} {len(t):5d} {statistics.mean(t):8.2f} {p50:8.2f} {t[len(t) // 10]:8.2f} "
              f"{t[(len(t) * 9) // 10]:8.2f} {gb:9.1f}  {' + '.join(uniq)}")


def _kname(full: str) -> str:
    """Kernel name without its argument list, return type or anonymous namespace."""
    return full.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def cmd_kstats(a):
    stats = one(os.path.join(a.dir, "*kernel_stats.csv"))
    cnt = {}
    for d in a.pmc:
        f = one(os.path.join(d, "*counter_collection.csv"))
        for r in csv.DictReader(open(f)):
            key = (_kname(r["Kernel_Name"]), r["Counter_Name"])
            cnt.setdefault(key, []).append(float(r["Counter_Value"]))
    print(f"# {a.title}")
    for c in a.command:
        print(f"# command: {c}")
    print("# kernel                                              calls    avg_ms    min_ms    max_ms" +
          ("   counters (mean per dispatch; FETCH_SIZE and WRITE_SIZE in KiB)" if cnt else ""))
    for r in csv.DictReader(open(stats)):
        name = _kname(r["Name"])
        extra = "  ".join(f"{cn}={statistics.mean(v):.0f}" for (kn, cn), v in sorted(cnt.items()) if kn == name)
        print(f"{name[:50]:50s} {int(r['Calls']):7d} {float(r['AverageNs']) * 1e-6:9.4f} "
              f"{float(r['MinNs']) * 1e-6:9.4f} {float(r['MaxNs']) * 1e-6:9.4f}   {extra}")


def cmd_pmc(a):
    per = {}                                   # counter -> row -> [values]
    for d in a.dirs:
        f = one(os.path.join(d, "*counter_collection.csv"))
        rows = list(csv.DictReader(open(f)))
        for name in sorted({r["Counter_Name"] for r in rows}):
            sub = [r for r in rows if r["Counter_Name"] == name]
            lab, _ = label(sub, "Kernel_Name", "Dispatch_Id")
            per[name] = {row: [] for row in ROWS}
            for _, row, r in lab:
                if row in per[name]:
                    per[name][row].append(float(r["Counter_Value"]))
    names = sorted(per)
    print("# rocprofv3 --pmc counters of the bench step kernels (P=8, bf16 [16384 x 8192] per rank,")
    print("# [16384 x 16384] for the ubatch row),")
    print("# mean per dispatch over every dispatch of each run")
    for c in a.command:
        print(f"# command: {c}")
    print("# row       " + "  ".join(f"{n:>18s}" for n in names))
    for row in ROWS:
        vals = [statistics.mean(per[n][row]) if per[n][row] else float("nan") for n in names]
        print(f"{row:10s} " + "  ".join(f"{v:18.1f}" for v in vals))
    print("#")
    print("# derived, per dispatch: algorithmic bytes per vector-memory instruction (a 64-lane")
    print("# wavefront moving 16 bytes per lane = 1024), waves launched, L2 (TCC) hit rate")
    for row in ROWS:
        m = {n: (statistics.mean(per[n][row]) if per[n][row] else None) for n in names}
        out = [f"{row:10s}"]
        rd, wr = m.get("SQ_INSTS_VMEM_RD"), m.get("SQ_INSTS_VMEM_WR")
        if rd is not None and wr is not None and rd + wr > 0:
            out.append(f"bytes/VMEM-instr {ALGO[row] / (rd + wr):8.1f}")
        if m.get("SQ_WAVES") is not None:
            out.append(f"waves {m['SQ_WAVES']:10.0f}")
        hit, miss = m.get("TCC_HIT_sum"), m.get("TCC_MISS_sum")
        if hit is not None and miss is not None and hit + miss > 0:
            out.append(f"L2 hit rate {hit / (hit + miss):.3f}")
        print("  ".join(out))


def counters(d):
    f = one(os.path.join(d, "*counter_collection.csv"))
    rows = list(csv.DictReader(open(f)))
    lab, _ = label(rows, "Kernel_Name", "Dispatch_Id")
    per = {r: [] for r in ROWS}
    for _, row, r in lab:
        if row in per:
            per[row].append(float(r["Counter_Value"]) * 1024.0)
    copy = [float(r["Counter_Value"]) * 1024.0 for r in rows if "k_copy" in r["Kernel_Name"]]
    if not copy:
        raise SystemExit(f"{f}: no calibration copy dispatches")
    return {k: statistics.mean(v) for k, v in per.items()}, statistics.mean(copy), rows[0]["Counter_Name"]


def cmd_traffic(a):
    fetch, fcopy, fname = counters(a.fetch_dir)
    write, wcopy, wname = counters(a.write_dir)
    fs, ws = a.calib_bytes / fcopy, a.calib_bytes / wcopy
    print("# HBM traffic per launch of the bench step kernels (P=8, bf16 [16384 x 8192] per rank,")
    print("# [16384 x 16384] for the ubatch row)")
    print(f"# fetch command: {a.command_fetch}")
    print(f"# write command: {a.command_write}")
    print(f"# counters: {fname} and {wname}, KiB per dispatch, averaged over every dispatch of the run;")
    print(f"# scaled by the plain copy of {a.calib_bytes} B: fetch x{fs:.5f}, write x{ws:.5f}")
    print(f"source_sha256: {sources_sha256()}")
    print(f"fetch_scale: {fs:.6f}")
    print(f"write_scale: {ws:.6f}")
    for row in ROWS:
        fb, wb = fetch[row] * fs, write[row] * ws
        print(f"{row}.fetch_bytes_per_launch: {fb:.0f}")
        print(f"{row}.write_bytes_per_launch: {wb:.0f}")
        print(f"{row}.hbm_bytes_per_launch: {fb + wb:.0f}")
        print(f"{row}.algorithmic_bytes_per_launch: {ALGO[row]}")
        print(f"{row}.traffic_over_algorithmic: {(fb + wb) / ALGO[row]:.4f}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--warmup", type=int, default=2)
    s.add_argument("--command", default="")
    ks = sub.add_parser("kstats")
    ks.add_argument("dir")
    ks.add_argument("--pmc", action="append", default=[])
    ks.add_argument("--title", default="rocprofv3 per-kernel statistics")
    ks.add_argument("--command", action="append", default=[])
    pm = sub.add_parser("pmc")
    pm.add_argument("dirs", nargs="+")
    pm.add_argument("--command", action="append", default=[])
    d = sub.add_parser("decode")
    d.add_argument("dir")
    d.add_argument("plan")
    d.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--calib-bytes", type=float, default=float(1 << 30))
    t.add_argument("--command-fetch", default="")
    t.add_argument("--command-write", default="")
    a = ap.parse_args(argv)
    return {"stats": cmd_stats, "decode": cmd_decode, "traffic": cmd_traffic, "pmc": cmd_pmc,
            "kstats": cmd_kstats}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
