"""The C-ABI from plain C.

tests/c_abi_check.c (built by __graft_entry__.build() as
tests/libcabicheck.so) is C99 code that allocates with the HIP C API, calls
the one-shot, both two-stage modes, pack / recursive doubling (three modes) /
unpack and the two-stream ubatch reduce through include/ar.h, and checks
every result against the exact integer sum it computes itself (small-integer
inputs, so every order of the additions gives the same bf16 result).  It runs
in this process: Python only calls it and reads its one-line report.
"""
import ctypes
import os

import pytest
import torch  # loads the HIP runtime the other tests use before the C code does

import tensor_all_reduce_amd as tar
from gpu_util import note

pytestmark = pytest.mark.gpu

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcabicheck.so")


def test_c_abi_from_plain_c():
    assert os.path.exists(PATH), f"{PATH} is not built; run __graft_entry__.build()"
    torch.cuda.init()
    tar.lib()
    L = ctypes.CDLL(PATH)
    L.c_abi_check.restype = ctypes.c_int
    L.c_abi_check.argtypes = []
    L.c_abi_check_message.restype = ctypes.c_char_p
    L.c_abi_check_message.argtypes = []
    note("plain-C check of the C-ABI")
    rc = L.c_abi_check()
    msg = L.c_abi_check_message().decode()
    print(msg)
    assert rc == 0, msg
