"""C-ABI host logic on the CPU: the library loads, exports every symbol that
include/ar.h declares, and rejects bad arguments before any HIP call.

No call here reaches a kernel launch: every call either fails validation or
has n == 0, both of which return before the library touches the device.
"""
import ctypes
import os
import re
import subprocess

import pytest

import tensor_all_reduce_amd as tar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ar.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["ar_reduce_oneshot", "ar_reduce_2stage", "ar_pack_fused", "ar_unpack_fused",
                 "ar_rd_schedule", "ar_reduce_ubatch", "ar_status_str", "ar_version", "ar_err_init",
                 "ar_unpack_fused_wait", "ar_reduce_ubatch_flags", "ar_quantize_fp8", "ar_reduce_fp8"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(tar.lib_path), "build first: python __graft_entry__.py"
    out = subprocess.run(["nm", "-D", "--defined-only", tar.lib_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(ar_[a-z0-9_]+)$", out, flags=re.M))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    L = tar.lib()
    for f in declared_functions():
        assert hasattr(L, f)


def test_header_constants_match_binding():
    src = open(HEADER).read()
    for name, val in re.findall(r"#define\s+(AR_[A-Z0-9_]+)\s+(-?\d+)", src):
        assert getattr(tar, name) == int(val), name


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-x", "c", "-std=c99", "-fsyntax-only", "-Wall", "-Werror", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings_and_version():
    assert tar.ar_status_str(0) == "AR_OK"
    for code in (-1, -2, -3, -4, -5, -6):
        assert tar.ar_status_str(code).startswith("AR_ERR_")
    assert tar.ar_status_str(123) == "AR_ERR_UNKNOWN"
    assert tar.ar_version() >= 10000


# ---------------------------------------------------------------- validation (no device access)

vp = ctypes.c_void_p
A = 0x10000000          # fake, 16-byte aligned "device" addresses: never dereferenced
B = 0x20000000
C = 0x30000000


def arr(*ptrs):
    return (vp * len(ptrs))(*ptrs)


def test_oneshot_validation():
    L = tar.lib()
    ins = arr(A, B)
    assert L.ar_reduce_oneshot(None, 2, C, 8, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_oneshot(ins, 0, C, 8, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_oneshot(arr(*([A] * 9)), 9, C, 8, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_oneshot(ins, 2, None, 8, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_oneshot(arr(A + 2, B), 2, C, 8, None) == tar.AR_ERR_ALIGN
    assert L.ar_reduce_oneshot(ins, 2, C + 8, 8, None) == tar.AR_ERR_ALIGN
    # partial overlap of the output with an input
    assert L.ar_reduce_oneshot(ins, 2, A + 16, 64, None) == tar.AR_ERR_ALIAS
    # exact in place and n == 0 are accepted without touching the device
    assert L.ar_reduce_oneshot(ins, 2, A, 0, None) == tar.AR_OK
    assert L.ar_reduce_oneshot(arr(A, A), 2, C, 0, None) == tar.AR_OK


def test_2stage_validation():
    L = tar.lib()
    ins = arr(A, B)
    assert L.ar_reduce_2stage(ins, None, 2, 8, None, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_2stage(ins, arr(C, None), 2, 8, None, None) == tar.AR_ERR_INVALID
    # two outputs overlapping each other
    assert L.ar_reduce_2stage(ins, arr(C, C + 16), 2, 64, None, None) == tar.AR_ERR_ALIAS
    assert L.ar_reduce_2stage(ins, arr(C, C), 2, 64, None, None) == tar.AR_ERR_ALIAS
    # scratch overlapping an output or input
    assert L.ar_reduce_2stage(ins, arr(C, C + 4096), 2, 64, C + 32, None) == tar.AR_ERR_ALIAS
    assert L.ar_reduce_2stage(ins, arr(C, C + 4096), 2, 64, A, None) == tar.AR_ERR_ALIAS
    assert L.ar_reduce_2stage(ins, arr(C, C + 4096), 2, 64, C + 8200, None) == tar.AR_ERR_ALIGN
    # in place (outs == ins) is fine
    assert L.ar_reduce_2stage(ins, arr(A, B), 2, 0, None, None) == tar.AR_OK


def test_bounded_ubatch_shape_and_flags_validation():
    L = tar.lib()
    K = tar.AR_KERNEL_UBATCH_BOUNDED
    default = tar.ar_get_launch_shape(K)
    assert default[0] in (256, 512, 1024) and 1 <= default[4] <= 8
    # the bounded kind takes 256..1024 lanes and a footprint of 1..8 eighths
    assert L.ar_set_launch_shape(K, 1024, 1, 1, 1, 8) == tar.AR_OK
    assert L.ar_set_launch_shape(K, 512, 1, 1, 1, 0) == tar.AR_ERR_INVALID
    assert L.ar_set_launch_shape(K, 512, 1, 1, 1, 9) == tar.AR_ERR_INVALID
    assert L.ar_set_launch_shape(K, 64, 1, 1, 1, 4) == tar.AR_ERR_INVALID
    # the other kinds keep their limits
    assert L.ar_set_launch_shape(tar.AR_KERNEL_UBATCH, 512, 1, 1, 1, 4) == tar.AR_ERR_INVALID
    assert L.ar_set_launch_shape(K, *default) == tar.AR_OK
    # completion flags have no bounded form: rejected before any device work
    ins, outs = arr(A, B), arr(C, C + 4096)
    done, tiles = ctypes.c_void_p(0x40000000), ctypes.c_void_p(0x40001000)
    rc = L.ar_reduce_ubatch_flags(ins, outs, 2, 4, 8, 1, None, 16, tar.AR_VARIANT_2STAGE | tar.AR_UBATCH_BOUNDED,
                                  arr(None), done, tiles, 64, 1)
    assert rc == tar.AR_ERR_UNSUPPORTED
    assert L.ar_reduce_ubatch(ins, outs, 2, 4, 8, 1, None, 16, 0x200, arr(None)) == tar.AR_ERR_INVALID


def test_2stage_static_validation():
    L = tar.lib()
    ins = arr(A, B)
    big = tar.AR_STATIC_SCRATCH_ELEMS
    assert L.ar_reduce_2stage_static(ins, None, 2, 8, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_2stage_static(ins, arr(C, C + 16), 2, 64, None) == tar.AR_ERR_ALIAS
    assert L.ar_reduce_2stage_static(ins, arr(C + 8, C + 4096), 2, 64, None) == tar.AR_ERR_ALIGN
    # beyond the static scratch: rejected before any device work
    assert L.ar_reduce_2stage_static(ins, arr(A, B), 2, big + 8, None) == tar.AR_ERR_SIZE
    assert tar.ar_status_str(tar.AR_ERR_SIZE).startswith("AR_ERR_SIZE")
    assert L.ar_reduce_2stage_static(ins, arr(A, B), 2, 0, None) == tar.AR_OK


def test_pack_unpack_validation():
    L = tar.lib()
    assert L.ar_pack_fused(A, B, 7, 1, None) == tar.AR_ERR_INVALID           # odd n
    assert L.ar_pack_fused(A, A + 16, 64, 1, None) == tar.AR_ERR_ALIAS
    assert L.ar_pack_fused(A + 4, B, 8, 1, None) == tar.AR_ERR_ALIGN
    assert L.ar_pack_fused(A, B, 0, 1, None) == tar.AR_OK
    assert L.ar_unpack_fused(A, B, 8, 1, None, None) == tar.AR_ERR_INVALID  # no error record
    assert L.ar_unpack_fused(A, B, 8, 1, C + 4, None) == tar.AR_ERR_ALIGN
    assert L.ar_unpack_fused(A, B, 8, 1, A + 8, None) == tar.AR_ERR_ALIAS
    assert L.ar_unpack_fused(A, B, 0, 1, C, None) == tar.AR_OK


def test_unpack_wait_validation():
    L = tar.lib()
    assert L.ar_unpack_fused_wait(A, B, 8, 1, 0, C, None) == tar.AR_ERR_INVALID   # max_spins 0
    assert L.ar_unpack_fused_wait(A, B, 7, 1, 5, C, None) == tar.AR_ERR_INVALID   # odd n
    assert L.ar_unpack_fused_wait(A, B, 8, 1, 5, None, None) == tar.AR_ERR_INVALID
    assert L.ar_unpack_fused_wait(A, B + 2, 8, 1, 5, C, None) == tar.AR_ERR_ALIGN
    assert L.ar_unpack_fused_wait(A, A + 16, 8, 1, 5, C, None) == tar.AR_ERR_ALIAS
    assert L.ar_unpack_fused_wait(A, B, 0, 1, 5, C, None) == tar.AR_OK


def test_rd_validation():
    L = tar.lib()
    ins3 = arr(A, A + 0x1000, A + 0x2000)
    outs3 = arr(B, B + 0x1000, B + 0x2000)
    assert L.ar_rd_schedule(ins3, outs3, 3, 8, 0, None, 0, C, None) == tar.AR_ERR_UNSUPPORTED
    ins = arr(*[A + 0x1000 * i for i in range(4)])
    outs = arr(*[B + 0x1000 * i for i in range(4)])
    assert L.ar_rd_schedule(ins, outs, 4, 7, 0, None, 0, C, None) == tar.AR_ERR_INVALID
    assert L.ar_rd_schedule(ins, outs, 4, 8, 0, None, 3, C, None) == tar.AR_ERR_UNSUPPORTED
    assert L.ar_rd_schedule(ins, outs, 4, 8, 0, None, 8, C, None) == tar.AR_ERR_INVALID
    assert L.ar_rd_schedule(ins, outs, 4, 8, 0, None, tar.AR_RD_STAGED, C, None) == tar.AR_ERR_INVALID
    assert L.ar_rd_schedule(ins, outs, 4, 8, 0, A, tar.AR_RD_STAGED, C, None) == tar.AR_ERR_ALIAS
    assert L.ar_rd_schedule(ins, outs, 4, 8, 0, C - 64, tar.AR_RD_STAGED, C, None) == tar.AR_ERR_ALIAS
    assert L.ar_rd_schedule(ins, outs, 4, 0, 0, C + 4096, tar.AR_RD_STAGED, C, None) == tar.AR_OK
    assert L.ar_rd_schedule(ins, ins, 4, 0, 0, None, 0, C, None) == tar.AR_OK   # in place


def test_ranges_near_top_of_address_space():
    """A range whose end would wrap past 2^64 still overlaps what lies above
    its start (the end saturates), so the alias check cannot be bypassed."""
    L = tar.lib()
    top = 2 ** 64 - 0x10000
    n = 2 ** 61                                   # 2n bytes run past the top
    assert L.ar_reduce_oneshot(arr(top, B), 2, top + 0x8000, n, None) == tar.AR_ERR_ALIAS
    assert L.ar_pack_fused(top, top + 0x8000, n, 1, None) == tar.AR_ERR_ALIAS


def test_ubatch_validation():
    L = tar.lib()
    ins = arr(A, B)
    outs = arr(C, C + 0x100000)
    streams = arr(None, None)
    ub = (ctypes.c_size_t * 2)(3, 3)
    assert L.ar_reduce_ubatch(ins, outs, 2, 4, 8, 2, ub, 4096, 1, streams) == tar.AR_ERR_INVALID
    assert L.ar_reduce_ubatch(ins, outs, 2, 4, 8, 2, None, 4008, 1, streams) == tar.AR_ERR_INVALID
    assert L.ar_reduce_ubatch(ins, outs, 2, 4, 8, 2, None, 0, 1, streams) == tar.AR_ERR_INVALID
    assert L.ar_reduce_ubatch(ins, outs, 2, 4, 8, 0, None, 4096, 1, streams) == tar.AR_ERR_INVALID
    assert L.ar_reduce_ubatch(ins, outs, 2, 4, 8, 2, None, 4096, 7, streams) == tar.AR_ERR_INVALID
    assert L.ar_reduce_ubatch(ins, outs, 2, 4, 8, 2, None, 4096, 1, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_ubatch(ins, arr(C, C + 16), 2, 4, 8, 2, None, 4096, 1, streams) == tar.AR_ERR_ALIAS
    # one-shot ignores outs[1]
    assert L.ar_reduce_ubatch(ins, arr(C, None), 2, 0, 8, 2, None, 4096, 0, streams) == tar.AR_OK


def test_ubatch_flags_validation():
    L = tar.lib()
    ins = arr(A, B)
    outs = arr(C, C + 0x100000)
    streams = arr(None, None)
    D = 0x40000000
    T = 0x40010000
    args = lambda done, tiles, nf, epoch: (ins, outs, 2, 4, 8, 2, None, 16, 1, streams, done, tiles, nf, epoch)
    # 4 rows x 8 = 32 elements, 16-byte chunks = 8 elements: 2 ubatches x 2 chunks
    assert L.ar_reduce_ubatch_flags(*args(None, T, 4, 1)) == tar.AR_ERR_INVALID
    assert L.ar_reduce_ubatch_flags(*args(D, None, 4, 1)) == tar.AR_ERR_INVALID
    assert L.ar_reduce_ubatch_flags(*args(D, T, 4, 0)) == tar.AR_ERR_INVALID      # epoch 0
    assert L.ar_reduce_ubatch_flags(*args(D, T, 3, 1)) == tar.AR_ERR_INVALID      # too short
    assert L.ar_reduce_ubatch_flags(*args(D + 2, T, 4, 1)) == tar.AR_ERR_ALIGN
    assert L.ar_reduce_ubatch_flags(*args(D, D + 8, 4, 1)) == tar.AR_ERR_ALIAS    # arrays overlap
    assert L.ar_reduce_ubatch_flags(*args(C, T, 4, 1)) == tar.AR_ERR_ALIAS        # flags over an output
    assert tar.ubatch_chunk_count(4, 8, 2, None, 16) == 4
    assert tar.ubatch_chunk_count(16384, 16384, 2, None, 1 << 20) == 512


def test_fp8_validation():
    L = tar.lib()
    xs = arr(A, B)
    codes = arr(C, C + 0x1000)
    scales = arr(C + 0x2000, C + 0x2001)          # one byte each for n = 32: any alignment
    # n = 32: codes 32 bytes, scales 1 byte; n = 0 passes every check and launches nothing
    assert L.ar_quantize_fp8(xs, codes, scales, 2, 0, None) == tar.AR_OK
    assert L.ar_quantize_fp8(None, codes, scales, 2, 32, None) == tar.AR_ERR_INVALID
    assert L.ar_quantize_fp8(xs, codes, scales, 0, 32, None) == tar.AR_ERR_INVALID
    assert L.ar_quantize_fp8(xs, codes, scales, 9, 32, None) == tar.AR_ERR_INVALID
    assert L.ar_quantize_fp8(xs, arr(C, None), scales, 2, 32, None) == tar.AR_ERR_INVALID
    assert L.ar_quantize_fp8(xs, arr(C + 8, C + 0x1000), scales, 2, 32, None) == tar.AR_ERR_ALIGN
    assert L.ar_quantize_fp8(arr(A + 2, B), codes, scales, 2, 32, None) == tar.AR_ERR_ALIGN
    assert L.ar_quantize_fp8(xs, arr(C, C + 16), scales, 2, 32, None) == tar.AR_ERR_ALIAS   # codes overlap
    assert L.ar_quantize_fp8(xs, codes, arr(C + 0x2000, C + 0x2000), 2, 32, None) == tar.AR_ERR_ALIAS
    assert L.ar_quantize_fp8(xs, codes, arr(C + 31, C + 0x2001), 2, 32, None) == tar.AR_ERR_ALIAS  # scale in codes
    assert L.ar_quantize_fp8(xs, arr(A + 32, C), scales, 2, 32, None) == tar.AR_ERR_ALIAS    # codes over input
    outs = arr(A, B)
    assert L.ar_reduce_fp8(codes, scales, 2, outs, 2, 0, None) == tar.AR_OK
    assert L.ar_reduce_fp8(codes, scales, 2, outs, 3, 32, None) == tar.AR_ERR_INVALID       # n_out not 1 or P
    assert L.ar_reduce_fp8(codes, scales, 2, outs, 0, 32, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_fp8(codes, scales, 0, outs, 1, 32, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_fp8(None, scales, 2, outs, 1, 32, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_fp8(codes, arr(C + 0x2000, None), 2, outs, 1, 32, None) == tar.AR_ERR_INVALID
    assert L.ar_reduce_fp8(arr(C + 4, C + 0x1000), scales, 2, outs, 1, 32, None) == tar.AR_ERR_ALIGN
    assert L.ar_reduce_fp8(codes, scales, 2, arr(A + 2, B), 1, 32, None) == tar.AR_ERR_ALIGN
    assert L.ar_reduce_fp8(codes, scales, 2, arr(A, A + 32), 2, 32, None) == tar.AR_ERR_ALIAS  # outputs overlap
    assert L.ar_reduce_fp8(codes, scales, 2, arr(C, B), 2, 32, None) == tar.AR_ERR_ALIAS      # output over codes
    assert L.ar_reduce_fp8(codes, scales, 2, arr(C + 0x1FF0, B), 2, 32, None) == tar.AR_ERR_ALIAS  # over a scale
    assert tar.fp8_scale_count(0) == 0 and tar.fp8_scale_count(32) == 1 and tar.fp8_scale_count(33) == 2


def test_err_init_validation():
    L = tar.lib()
    assert L.ar_err_init(None, None) == tar.AR_ERR_INVALID
    assert L.ar_err_init(C + 4, None) == tar.AR_ERR_ALIGN


def test_binding_raises_on_error():
    with pytest.raises(tar.ARError) as ei:
        tar._check(tar.AR_ERR_ALIAS, "ar_reduce_oneshot")
    assert ei.value.code == tar.AR_ERR_ALIAS


def test_launch_shape_roundtrip_and_validation():
    L = tar.lib()
    for kind in [k for k in range(tar.AR_KERNEL_2STAGE_INPLACE_SMALL + 1) if k != tar.AR_KERNEL_UBATCH_BOUNDED]:
        before = tar.ar_get_launch_shape(kind)
        tar.ar_set_launch_shape(kind, 128, 2, 0, 1, 7)
        assert tar.ar_get_launch_shape(kind) == (128, 2, 0, 1, 7)
        tar.ar_set_launch_shape(kind, *before)
        assert tar.ar_get_launch_shape(kind) == before
    assert L.ar_set_launch_shape(20, 64, 1, 1, 1, 0) == tar.AR_ERR_INVALID   # the bounded grid: 256..1024 lanes
    assert L.ar_set_launch_shape(tar.AR_KERNEL_2STAGE_INPLACE_SMALL + 1, 64, 1, 1, 1, 0) == tar.AR_ERR_INVALID
    assert L.ar_set_launch_shape(0, 96, 1, 1, 1, 0) == tar.AR_ERR_INVALID
    assert L.ar_set_launch_shape(0, 64, 3, 1, 1, 0) == tar.AR_ERR_INVALID
    assert L.ar_set_launch_shape(0, 64, 1, 2, 1, 0) == tar.AR_ERR_INVALID
    assert L.ar_set_launch_shape(0, 64, 1, 1, 1, 65) == tar.AR_ERR_INVALID
    assert L.ar_get_launch_shape(0, None, None, None, None, None) == tar.AR_ERR_INVALID


class _FakeDevTensor:
    """Stands in for a device tensor in the binding's checks (no GPU here)."""

    is_cuda = True

    def __init__(self, ptr: int, n: int, elem_size: int = 2):
        self._ptr, self._n, self._es = ptr, n, elem_size

    def is_contiguous(self):
        return True

    def element_size(self):
        return self._es

    def numel(self):
        return self._n

    def data_ptr(self):
        return self._ptr


def test_prepare_marshals_once_and_calls_later():
    import weakref

    n = 4096
    ins = [_FakeDevTensor(0x10000000 + i * 0x100000, n) for i in range(8)]
    outs = [_FakeDevTensor(0x20000000 + i * 0x100000, n) for i in range(8)]
    outs[5] = _FakeDevTensor(0x20000000 + 5 * 0x100000 + 2, n)          # not 16-byte aligned
    probe = weakref.ref(outs[5])
    h = tar.prepare(tar.ar_reduce_2stage, ins, outs, stream=0)      # would raise here if it made the call
    assert isinstance(h, tar.Prepared) and h.name == "ar_reduce_2stage"
    assert getattr(tar._tls, "capture", None) is None
    for _ in range(2):
        with pytest.raises(tar.ARError) as ei:
            h()
        assert ei.value.code == tar.AR_ERR_ALIGN
    del outs
    assert probe() is not None                     # the handle keeps its buffers alive
    del h, ei                                      # (the traceback refers to the handle too)
    assert probe() is None


def test_prepare_validates_like_the_wrapper():
    ins = [_FakeDevTensor(0x10000000 + i * 0x100000, 100) for i in range(8)]
    outs = [_FakeDevTensor(0x20000000 + i * 0x100000, 99) for i in range(8)]
    with pytest.raises(ValueError, match="outs"):
        tar.prepare(tar.ar_reduce_2stage, ins, outs, stream=0)
    assert getattr(tar._tls, "capture", None) is None
    with pytest.raises(ValueError, match="one output per rank"):
        tar.prepare(tar.ar_reduce_2stage, ins, ins[:7], stream=0)


def test_prepare_takes_device_calls_only():
    before = tar.ar_get_launch_shape(tar.AR_KERNEL_ONESHOT)
    with pytest.raises(ValueError, match="device call"):
        tar.prepare(tar.ar_set_launch_shape, tar.AR_KERNEL_ONESHOT, 64, 1, 0, 0, 0)
    assert tar.ar_get_launch_shape(tar.AR_KERNEL_ONESHOT) == before
    with pytest.raises(ValueError, match="device call"):
        tar.prepare(print, "x")


def test_prepare_every_device_call():
    """Each device call of the binding prepares (its marshalled arguments
    match the C signature's count and types) and its handle reaches the C
    validation, which rejects the misaligned stand-in buffers."""
    base = [0x30000000]

    def t(n, es=2):
        base[0] += 0x1000000
        return _FakeDevTensor(base[0] + 2, n, es)             # every buffer misaligned

    P, n, rows, hidden = 8, 4096, 4, 1024
    ins, outs = [t(n) for _ in range(P)], [t(n) for _ in range(P)]
    words, wout = [t(n // 2, 8) for _ in range(P)], [t(n // 2, 8) for _ in range(P)]
    err, x = t(2, 8), t(n)
    codes, scales = [t(n, 1) for _ in range(P)], [t(tar.fp8_scale_count(n), 1) for _ in range(P)]
    nch = tar.ubatch_chunk_count(rows, hidden)
    calls = [
        (tar.ar_reduce_oneshot, (ins, outs[0]), {"stream": 0}),
        (tar.ar_reduce_2stage, (ins, outs), {"stream": 0}),
        (tar.ar_reduce_2stage, (ins, outs), {"scratch": t(n), "stream": 0}),
        (tar.ar_reduce_2stage_static, (ins, outs), {"stream": 0}),
        (tar.ar_pack_fused, (x, words[0], 1), {"stream": 0}),
        (tar.ar_unpack_fused, (words[0], x, 1, err), {"stream": 0}),
        (tar.ar_unpack_fused_wait, (words[0], x, 1, err), {"stream": 0}),
        (tar.ar_rd_schedule, (words, wout, 1, err), {"stream": 0}),
        (tar.ar_reduce_ubatch, (ins, outs, rows, hidden), {"streams": [0, 0]}),
        (tar.ar_reduce_ubatch_flags, (ins, outs, rows, hidden, t(nch, 4), t(nch, 4), 1), {"streams": [0, 0]}),
        (tar.ar_quantize_fp8, (ins, codes, scales), {"stream": 0}),
        (tar.ar_reduce_fp8, (codes, scales, outs), {"stream": 0}),
        (tar.ar_err_init, (err,), {"stream": 0}),
    ]
    assert {c[0] for c in calls} == tar._PREPARABLE
    for func, a, k in calls:
        h = tar.prepare(func, *a, **k)
        assert h.name == func.__name__
        with pytest.raises(tar.ARError) as ei:
            h()
        assert ei.value.code in (tar.AR_ERR_ALIGN, tar.AR_ERR_INVALID), func.__name__
