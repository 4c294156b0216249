"""Host-side measurement logic on the CPU: the profile summariser's dispatch
labelling and counter scaling, the bench's source-hash gate on the traffic
record, and the bench's refusal of more than one GPU.  No GPU is touched."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench                                     # noqa: E402
from tensor_all_reduce_amd import profsum        # noqa: E402

NAMES = {"oneshot": "void ar::k_reduce<8, 1, 1, true, true, false>(ar::InPtrs)",
         "2stage": "void ar::k_reduce<8, 8, 2, true, true, false>(ar::InPtrs)",
         "pack": "void ar::k_pack<true, false>(void const*)",
         "err_init": "ar::k_err_init(unsigned long*)",
         "rd": "void ar::k_rd_fused<8, 1, true, true, true>(ar::WordIn)",
         "unpack": "void ar::k_unpack<false, true>(unsigned long const*)",
         "ubatch": "void ar::k_reduce<8, 8, 1, true, true, false>(ar::InPtrs)"}


def fake_dispatches(steps, with_copy=False):
    rows, d = [], 0
    for s in range(steps):
        for row in profsum.STEP:
            d += 1
            rows.append({"Dispatch_Id": str(d), "Kernel_Name": NAMES[row], "row": row, "step": s})
            if row == "rd" and s == 0:
                d += 1                          # a non-library kernel in between is ignored
                rows.append({"Dispatch_Id": str(d), "Kernel_Name": "at::native::fill_kernel", "row": None,
                             "step": s})
    if with_copy:
        for _ in range(3):
            d += 1
            rows.append({"Dispatch_Id": str(d), "Kernel_Name": "(anonymous namespace)::k_copy(u32x4*)",
                         "row": None, "step": None})
    return rows


def test_label_follows_the_step_sequence():
    rows = fake_dispatches(3)
    lab, steps = profsum.label(rows, "Kernel_Name", "Dispatch_Id")
    assert steps == 3 and len(lab) == 3 * len(profsum.STEP)
    for s, row, r in lab:
        assert r["row"] == row and r["step"] == s


def test_label_rejects_a_sequence_that_does_not_match():
    rows = fake_dispatches(2)
    rows[1]["Kernel_Name"] = NAMES["pack"]      # the 2stage dispatch replaced by another kernel
    with pytest.raises(SystemExit):
        profsum.label(rows, "Kernel_Name", "Dispatch_Id")


def write_counters(d, name, per_row_kib, copy_kib):
    os.makedirs(d)
    with open(os.path.join(d, "bench_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in fake_dispatches(2, with_copy=True):
            row = r["row"]
            if row is None and "k_copy" in r["Kernel_Name"]:
                v = copy_kib
            else:
                v = per_row_kib.get(row, 1.0)
            w.writerow({"Dispatch_Id": r["Dispatch_Id"], "Kernel_Name": r["Kernel_Name"],
                        "Counter_Name": name, "Counter_Value": v})


def test_traffic_scales_by_the_copy_and_gates_on_sources(tmp_path, capsys):
    # each row reads and writes half its algorithmic bytes; the fetch counter
    # sees half of what is read (as FETCH_SIZE does with non-temporal loads),
    # the write counter all of what is written; counters are in KiB
    B = profsum.B
    fetch = {r: profsum.ALGO[r] / 2 / 2 / 1024 for r in profsum.ROWS}
    write = {r: profsum.ALGO[r] / 2 / 1024 for r in profsum.ROWS}
    write_counters(str(tmp_path / "f"), "FETCH_SIZE", fetch, (1 << 30) / 2 / 1024)
    write_counters(str(tmp_path / "w"), "WRITE_SIZE", write, (1 << 30) / 1024)
    profsum.main(["traffic", str(tmp_path / "f"), str(tmp_path / "w"), "--calib-bytes", str(float(1 << 30))])
    out = capsys.readouterr().out
    rec = dict(l.split(": ", 1) for l in out.splitlines() if ": " in l and not l.startswith("#"))
    assert abs(float(rec["fetch_scale"]) - 2.0) < 1e-9 and abs(float(rec["write_scale"]) - 1.0) < 1e-9
    for r in profsum.ROWS:
        assert abs(float(rec[f"{r}.traffic_over_algorithmic"]) - 1.0) < 1e-4
    # the bench uses the record only while the kernel sources are unchanged
    path = tmp_path / "traffic.txt"
    path.write_text(out)
    assert bench.load_traffic("rd", bench.KERNEL_SOURCES, str(path)) == pytest.approx(profsum.ALGO["rd"], rel=1e-6)
    stale = out.replace(rec["source_sha256"], "0" * 64)
    path.write_text(stale)
    assert bench.load_traffic("rd", bench.KERNEL_SOURCES, str(path)) is None
    assert B == 2 * 16384 * 8192


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 4 and "one GPU" in msg["error"]
