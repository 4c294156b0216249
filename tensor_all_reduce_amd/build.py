"""Build the gfx950 HIP library in-tree (``tensor_all_reduce_amd/libarcore.so``).

Plain hipcc invocations, no JIT: the built library sits next to this file so
it travels with the source tree.  ``build()`` always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libarcore.so")
BENCH_LIB = os.path.join(HERE, "libarbench.so")
SOURCES = ["ar_api.hip", "ar_reduce.hip", "ar_fused.hip", "ar_fp8.hip"]
BENCH_SOURCES = ["ar_bench.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -O3 without fast-math: IEEE binary32 adds, subnormals kept, no
# reassociation.  Packed-fp32 VALU ops are switched off: the reduction gains
# nothing from them and their use is avoided on these parts.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(sources, verbose, jobs):
    objs, procs = [], []
    for src in sources:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
        if len(procs) >= jobs:
            p, c = procs.pop(0)
            if p.wait() != 0:
                raise RuntimeError("hipcc failed: " + " ".join(c))
    for p, c in procs:
        if p.wait() != 0:
            raise RuntimeError("hipcc failed: " + " ".join(c))
    return objs


def _link(objs, out, extra, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, *extra]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile libarcore.so (the library) and libarbench.so (timing helpers
    and a copy kernel used only by bench.py; linked against libarcore.so)."""
    objs = _compile(SOURCES + BENCH_SOURCES, verbose, jobs)
    _link(objs[: len(SOURCES)], LIB, [], verbose)
    _link(objs[len(SOURCES):], BENCH_LIB, ["-L", HERE, "-larcore", "-Wl,-rpath,$ORIGIN"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
