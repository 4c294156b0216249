"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/oracle_sanitize_main.c includes oracle/ar_oracle.c and calls every
oracle function on edge-case sizes with exactly sized buffers; built with
gcc -fsanitize=address,undefined and no recovery, any out-of-bounds access,
use after free or undefined arithmetic ends the run with a report."""
import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    flags = [f for f in oracle.GCC_FLAGS if f not in ("-shared", "-fPIC")]
    r = subprocess.run(["gcc", *flags, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-fno-omit-frame-pointer", os.path.join(HERE, "oracle_sanitize_main.c"), "-o", str(exe),
                        "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # the environment is passed through unchanged apart from the sanitizer
    # options; verify_asan_link_order=0 lets the run start when another
    # library is loaded ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "oracle sanitize run: ok" in run.stdout
