"""The compact small-message two-stage kernel's buffer offsets, on the host.

tests/offsets_check.cpp includes tensor_all_reduce_amd/csrc/ar_offsets.hpp
(the header that both the library's host code, to pack the offsets, and its
kernel, to rebuild the addresses, use) and checks the unit, the exact reach
limits (INT32_MAX and INT32_MIN units fit, one more does not), the 2^30 cap
on the unit, partial aliasing, every buffer count, and that every rebuilt
address is the original.  Built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, no recovery."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_offsets_pack_and_rebuild(tmp_path):
    exe = tmp_path / "offsets_check"
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "tensor_all_reduce_amd", "csrc"),
                        os.path.join(HERE, "offsets_check.cpp"), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "offsets check: ok" in run.stdout
