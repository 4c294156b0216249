"""MI355X (gfx950) multi-buffer all-reduce core: Python binding of libarcore.

A thin ctypes layer over the C-ABI in ``include/ar.h``.  Every function has
the C name and only marshals arguments: torch tensors become device
pointers and element counts, torch streams become ``hipStream_t`` handles.
All arithmetic runs in the HIP kernels of ``libarcore.so``; there is no
fallback of any kind.  If the library is missing, every call raises.

``prepare(func, *args, **kwargs)`` runs a device call's checks and
marshalling once and returns a handle that makes the same C-ABI call each
time it is called: for loops that pass the same buffers on every step.

bf16 buffers may be passed as ``torch.bfloat16`` or ``torch.int16`` /
``torch.uint16`` tensors (only the 16-bit patterns matter); payload words as
``torch.int64`` / ``torch.uint64`` tensors; error records as a 2-element
64-bit tensor.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Sequence

__all__ = [
    "ARError", "Prepared", "prepare", "lib", "lib_path", "ar_status_str", "ar_version", "ar_reduce_oneshot",
    "ar_reduce_2stage", "ar_reduce_2stage_static", "ar_pack_fused", "ar_unpack_fused", "ar_rd_schedule",
    "ar_reduce_ubatch", "ar_err_init", "rd_mailbox_words",
    "AR_OK", "AR_ERR_INVALID", "AR_ERR_ALIGN", "AR_ERR_ALIAS", "AR_ERR_UNSUPPORTED",
    "AR_ERR_HIP", "AR_ERR_SIZE", "AR_STATIC_SCRATCH_ELEMS", "AR_MAX_RANKS", "AR_VARIANT_ONESHOT", "AR_VARIANT_2STAGE", "AR_UBATCH_BOUNDED",
    "AR_RD_STAGED", "AR_RD_FP32_CARRY", "ar_set_launch_shape", "ar_get_launch_shape",
    "AR_KERNEL_ONESHOT", "AR_KERNEL_2STAGE", "AR_KERNEL_UBATCH", "AR_KERNEL_RS", "AR_KERNEL_AG",
    "AR_KERNEL_PACK", "AR_KERNEL_UNPACK", "AR_KERNEL_RD", "AR_KERNEL_RDSTEP", "AR_KERNEL_UNPACK_WAIT",
    "AR_KERNEL_UBATCH_FLAGS", "ar_unpack_fused_wait", "ar_reduce_ubatch_flags", "ubatch_chunk_count",
    "AR_KERNEL_QUANT_FP8", "AR_KERNEL_REDUCE_FP8", "AR_KERNEL_REDUCE_FP8_ALL", "ar_quantize_fp8", "ar_reduce_fp8", "fp8_scale_count",
    "AR_KERNEL_ONESHOT_SMALL", "AR_KERNEL_2STAGE_SMALL", "AR_KERNEL_RD_SMALL", "AR_KERNEL_RDSTEP_SMALL",
    "AR_KERNEL_PACK_SMALL", "AR_KERNEL_UNPACK_SMALL", "AR_KERNEL_UBATCH_BOUNDED",
    "AR_KERNEL_2STAGE_INPLACE_SMALL",
    "AR_SMALL_ELEMS",
    "FP8_BLOCK",
]

AR_OK = 0
AR_ERR_INVALID = -1
AR_ERR_ALIGN = -2
AR_ERR_ALIAS = -3
AR_ERR_UNSUPPORTED = -4
AR_ERR_HIP = -5
AR_ERR_SIZE = -6
AR_STATIC_SCRATCH_ELEMS = 16777216
AR_MAX_RANKS = 8
AR_VARIANT_ONESHOT = 0
AR_VARIANT_2STAGE = 1
AR_UBATCH_BOUNDED = 256
AR_RD_STAGED = 1
AR_RD_FP32_CARRY = 2
AR_KERNEL_ONESHOT = 0
AR_KERNEL_2STAGE = 1
AR_KERNEL_UBATCH = 2
AR_KERNEL_RS = 3
AR_KERNEL_AG = 4
AR_KERNEL_PACK = 5
AR_KERNEL_UNPACK = 6
AR_KERNEL_RD = 7
AR_KERNEL_RDSTEP = 8
AR_KERNEL_UNPACK_WAIT = 9
AR_KERNEL_UBATCH_FLAGS = 10
AR_KERNEL_QUANT_FP8 = 11
AR_KERNEL_REDUCE_FP8 = 12
AR_KERNEL_REDUCE_FP8_ALL = 13
AR_KERNEL_ONESHOT_SMALL = 14
AR_KERNEL_2STAGE_SMALL = 15
AR_KERNEL_RD_SMALL = 16
AR_KERNEL_RDSTEP_SMALL = 17
AR_KERNEL_PACK_SMALL = 18
AR_KERNEL_UNPACK_SMALL = 19
AR_KERNEL_UBATCH_BOUNDED = 20
AR_KERNEL_2STAGE_INPLACE_SMALL = 21
AR_SMALL_ELEMS = 2097152
FP8_BLOCK = 32                  # elements per power-of-two scale

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libarcore.so")
_lib = None

_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_u32 = ctypes.c_uint32


class ARError(RuntimeError):
    """A nonzero status from the C-ABI."""

    def __init__(self, code: int, func: str):
        self.code = code
        super().__init__(f"{func}: {ar_status_str(code)} ({code})")


def lib():
    """Load libarcore.so from this package directory (raises if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} is not built; run __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950)")
        L = ctypes.CDLL(lib_path)
        L.ar_status_str.restype = ctypes.c_char_p
        L.ar_status_str.argtypes = [ctypes.c_int]
        L.ar_version.restype = ctypes.c_int
        L.ar_version.argtypes = []
        L.ar_reduce_oneshot.restype = ctypes.c_int
        L.ar_reduce_oneshot.argtypes = [ctypes.POINTER(_vp), ctypes.c_int, _vp, _sz, _vp]
        L.ar_reduce_2stage.restype = ctypes.c_int
        L.ar_reduce_2stage.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.c_int, _sz,
                                       _vp, _vp]
        L.ar_reduce_2stage_static.restype = ctypes.c_int
        L.ar_reduce_2stage_static.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.c_int, _sz, _vp]
        L.ar_pack_fused.restype = ctypes.c_int
        L.ar_pack_fused.argtypes = [_vp, _vp, _sz, _u32, _vp]
        L.ar_unpack_fused.restype = ctypes.c_int
        L.ar_unpack_fused.argtypes = [_vp, _vp, _sz, _u32, _vp, _vp]
        L.ar_unpack_fused_wait.restype = ctypes.c_int
        L.ar_unpack_fused_wait.argtypes = [_vp, _vp, _sz, _u32, _u32, _vp, _vp]
        L.ar_rd_schedule.restype = ctypes.c_int
        L.ar_rd_schedule.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.c_int, _sz,
                                     _u32, _vp, ctypes.c_int, _vp, _vp]
        L.ar_reduce_ubatch.restype = ctypes.c_int
        L.ar_reduce_ubatch.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.c_int, _sz,
                                       _sz, ctypes.c_int, ctypes.POINTER(_sz), _sz, ctypes.c_int,
                                       ctypes.POINTER(_vp)]
        L.ar_reduce_ubatch_flags.restype = ctypes.c_int
        L.ar_reduce_ubatch_flags.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.c_int, _sz,
                                             _sz, ctypes.c_int, ctypes.POINTER(_sz), _sz, ctypes.c_int,
                                             ctypes.POINTER(_vp), _vp, _vp, _sz, _u32]
        L.ar_err_init.restype = ctypes.c_int
        L.ar_err_init.argtypes = [_vp, _vp]
        L.ar_quantize_fp8.restype = ctypes.c_int
        L.ar_quantize_fp8.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                      ctypes.c_int, _sz, _vp]
        L.ar_reduce_fp8.restype = ctypes.c_int
        L.ar_reduce_fp8.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.c_int,
                                    ctypes.POINTER(_vp), ctypes.c_int, _sz, _vp]
        L.ar_set_launch_shape.restype = ctypes.c_int
        L.ar_set_launch_shape.argtypes = [ctypes.c_int] * 6
        ip = ctypes.POINTER(ctypes.c_int)
        L.ar_get_launch_shape.restype = ctypes.c_int
        L.ar_get_launch_shape.argtypes = [ctypes.c_int, ip, ip, ip, ip, ip]
        _lib = L
    return _lib


def ar_status_str(code: int) -> str:
    return lib().ar_status_str(int(code)).decode()


def ar_version() -> int:
    return int(lib().ar_version())


# ---------------------------------------------------------------- marshalling

def _check(rc: int, func: str) -> None:
    if rc != AR_OK:
        raise ARError(rc, func)


_tls = threading.local()


def _call(name: str, *cargs) -> None:
    """Make one device call of the library with marshalled arguments, or,
    inside prepare(), record it instead of making it."""
    fn = getattr(lib(), name)
    slot = getattr(_tls, "capture", None)
    if slot is not None:
        slot.append((fn, name, cargs))
        return
    _check(fn(*cargs), name)


class Prepared:
    """One device call with its arguments checked and marshalled once.

    Calling it makes the same C-ABI call as the wrapper it was prepared from,
    with the same device pointers, sizes and stream, and raises ARError on a
    nonzero status.  It holds references to the tensors it was prepared
    with, so their storage stays allocated while the handle lives; their
    contents may change between calls (that is the point), their storage
    must not be replaced (``set_``, ``resize_``).  The stream is the one
    named at prepare time, or the current stream then if none was named.
    """

    __slots__ = ("_fn", "_name", "_args", "_refs")

    def __init__(self, fn, name: str, cargs: tuple, refs: tuple):
        if len(cargs) != len(fn.argtypes):
            raise TypeError(f"{name}: {len(cargs)} arguments for {len(fn.argtypes)} parameters")
        # plain ints become instances of the declared C types now, which
        # ctypes then passes through as they are (about 0.1 us a call)
        conv = tuple(t(a) if isinstance(a, int) else a for a, t in zip(cargs, fn.argtypes))
        self._fn, self._name, self._args, self._refs = fn, name, conv, refs

    @property
    def name(self) -> str:
        return self._name

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != AR_OK:
            raise ARError(rc, self._name)

    def __repr__(self) -> str:
        return f"<Prepared {self._name}>"


def prepare(func, *args, **kwargs) -> Prepared:
    """Check and marshal the arguments of one device call once.

    ``prepare(ar_reduce_2stage, ins, outs)`` validates ``ins`` and ``outs``
    exactly as ``ar_reduce_2stage(ins, outs)`` would (raising the same
    errors), queues nothing, and returns a Prepared handle whose call queues
    that work.  For loops that pass the same buffers on every step (a decode
    step's all-reduce): a wrapper call spends about 0.45 us per tensor in
    checks and pointer lookups, a prepared call none.  ``func`` is one of the
    device calls of this module."""
    if func not in _PREPARABLE:
        raise ValueError(f"prepare() takes a device call of this module, not {func!r}")
    slot = []
    _tls.capture = slot
    try:
        func(*args, **kwargs)
    finally:
        _tls.capture = None
    (fn, name, cargs), = slot
    return Prepared(fn, name, cargs, (args, kwargs))


def _dev_ptr(t, elem_size: int, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.element_size() != elem_size:
        raise ValueError(f"{name} must have {elem_size}-byte elements")
    return t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr_array(ptrs):
    arr = (_vp * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def _bufs(ts, elem_size: int, name: str, count: int | None = None):
    ptrs = []
    for i, t in enumerate(ts):
        if t is None:
            ptrs.append(None)
            continue
        if count is not None and t.numel() < count:
            raise ValueError(f"{name}[{i}] holds {t.numel()} elements, {count} needed")
        ptrs.append(_dev_ptr(t, elem_size, f"{name}[{i}]"))
    return ptrs


def ar_reduce_oneshot(ins: Sequence, out, n: int | None = None, stream=None) -> None:
    """out[:n] = sum of ins[p][:n] (binary32 accumulation in rank order, one bf16 rounding)."""
    n = ins[0].numel() if n is None else int(n)
    ip = _bufs(ins, 2, "ins", n)
    (op,) = _bufs([out], 2, "out", n)
    _call("ar_reduce_oneshot", _ptr_array(ip), len(ip), op, n, _stream(stream))


def ar_reduce_2stage(ins: Sequence, outs: Sequence, scratch=None, n: int | None = None,
                     stream=None) -> None:
    """Every outs[r][:n] = the one-shot sum; scratch given -> staged RS/AG.
    outs may be ins itself (in place: each rank's result in its own buffer)."""
    n = ins[0].numel() if n is None else int(n)
    ip = _bufs(ins, 2, "ins", n)
    op = _bufs(outs, 2, "outs", n)
    if len(op) != len(ip):
        raise ValueError("need one output per rank")
    sp = None if scratch is None else _bufs([scratch], 2, "scratch", n)[0]
    _call("ar_reduce_2stage", _ptr_array(ip), _ptr_array(op), len(ip), n, sp, _stream(stream))


def ar_reduce_2stage_static(ins: Sequence, outs: Sequence, n: int | None = None, stream=None) -> None:
    """The staged two-stage reduce through the library's static scratch (no
    allocation, no workspace argument); n <= AR_STATIC_SCRATCH_ELEMS."""
    n = ins[0].numel() if n is None else int(n)
    ip = _bufs(ins, 2, "ins", n)
    op = _bufs(outs, 2, "outs", n)
    if len(op) != len(ip):
        raise ValueError("need one output per rank")
    _call("ar_reduce_2stage_static", _ptr_array(ip), _ptr_array(op), len(ip), n, _stream(stream))


def ar_pack_fused(x, words, seq: int, n: int | None = None, stream=None) -> None:
    n = x.numel() if n is None else int(n)
    (xp,) = _bufs([x], 2, "x", n)
    (wp,) = _bufs([words], 8, "words", n // 2)
    _call("ar_pack_fused", xp, wp, n, int(seq) & 0xFFFFFFFF, _stream(stream))


def ar_unpack_fused(words, x, expected_seq: int, d_err, n: int | None = None, stream=None) -> None:
    n = x.numel() if n is None else int(n)
    (wp,) = _bufs([words], 8, "words", n // 2)
    (xp,) = _bufs([x], 2, "x", n)
    (ep,) = _bufs([d_err], 8, "d_err", 2)
    _call("ar_unpack_fused", wp, xp, n, int(expected_seq) & 0xFFFFFFFF, ep, _stream(stream))


def ar_unpack_fused_wait(words, x, expected_seq: int, d_err, max_spins: int = 1 << 20,
                         n: int | None = None, stream=None) -> None:
    """Unpack, waiting (at most max_spins polls per wavefront) for a
    concurrent producer to write payloads carrying expected_seq."""
    n = x.numel() if n is None else int(n)
    (wp,) = _bufs([words], 8, "words", n // 2)
    (xp,) = _bufs([x], 2, "x", n)
    (ep,) = _bufs([d_err], 8, "d_err", 2)
    _call("ar_unpack_fused_wait", wp, xp, n, int(expected_seq) & 0xFFFFFFFF, int(max_spins), ep,
          _stream(stream))


def rd_mailbox_words(P: int, n: int) -> int:
    """Mailbox size in payload words for ar_rd_schedule(..., AR_RD_STAGED)."""
    steps = {2: 1, 4: 2, 8: 3}[P]
    W = n // 2
    return P * (steps - 1) * (W + (W & 1))


def ar_rd_schedule(in_words: Sequence, out_words: Sequence, seq0: int, d_err, mailbox=None,
                   flags: int = 0, n: int | None = None, stream=None) -> None:
    n = 2 * in_words[0].numel() if n is None else int(n)
    ip = _bufs(in_words, 8, "in_words", n // 2)
    op = _bufs(out_words, 8, "out_words", n // 2)
    if len(op) != len(ip):
        raise ValueError("need one output payload per rank")
    mp = None
    if mailbox is not None:
        (mp,) = _bufs([mailbox], 8, "mailbox", rd_mailbox_words(len(ip), n) if len(ip) in (2, 4, 8) else 0)
    (ep,) = _bufs([d_err], 8, "d_err", 2)
    _call("ar_rd_schedule", _ptr_array(ip), _ptr_array(op), len(ip), n, int(seq0) & 0xFFFFFFFF,
          mp, int(flags), ep, _stream(stream))


def ar_reduce_ubatch(ins: Sequence, outs: Sequence, rows: int, hidden: int, n_ubatch: int = 2,
                     ubatch_rows: Sequence[int] | None = None, chunk_bytes: int = 1 << 20,
                     variant: int = AR_VARIANT_2STAGE, streams: Sequence | None = None) -> None:
    n = int(rows) * int(hidden)
    ip = _bufs(ins, 2, "ins", n)
    op = _bufs(outs, 2, "outs", n)
    if streams is None:
        streams = [None] * n_ubatch
    if len(streams) != n_ubatch:
        raise ValueError("need one stream per ubatch")
    sp = _ptr_array([_stream(s) for s in streams])
    ub = None
    if ubatch_rows is not None:
        if len(ubatch_rows) != n_ubatch:
            raise ValueError("need one row count per ubatch")
        ub = (_sz * n_ubatch)(*[int(r) for r in ubatch_rows])
    _call("ar_reduce_ubatch", _ptr_array(ip), _ptr_array(op), len(ip), int(rows), int(hidden),
          int(n_ubatch), ub, int(chunk_bytes), int(variant), sp)


def ubatch_chunk_count(rows: int, hidden: int, n_ubatch: int = 2, ubatch_rows=None,
                       chunk_bytes: int = 1 << 20) -> int:
    """Total chunks of a ubatch reduce (size of the flag arrays)."""
    if ubatch_rows is None:
        ubatch_rows = [rows // n_ubatch] * (n_ubatch - 1)
        ubatch_rows.append(rows - sum(ubatch_rows))
    ce = chunk_bytes // 2
    return sum((int(r) * hidden + ce - 1) // ce for r in ubatch_rows)


def ar_reduce_ubatch_flags(ins: Sequence, outs: Sequence, rows: int, hidden: int, chunk_done,
                           chunk_tiles, epoch: int, n_ubatch: int = 2,
                           ubatch_rows: Sequence[int] | None = None, chunk_bytes: int = 1 << 20,
                           variant: int = AR_VARIANT_2STAGE, streams: Sequence | None = None) -> None:
    """ar_reduce_ubatch that also publishes done[chunk] = epoch per chunk."""
    n = int(rows) * int(hidden)
    ip = _bufs(ins, 2, "ins", n)
    op = _bufs(outs, 2, "outs", n)
    if streams is None:
        streams = [None] * n_ubatch
    if len(streams) != n_ubatch:
        raise ValueError("need one stream per ubatch")
    sp = _ptr_array([_stream(s) for s in streams])
    ub = None
    if ubatch_rows is not None:
        if len(ubatch_rows) != n_ubatch:
            raise ValueError("need one row count per ubatch")
        ub = (_sz * n_ubatch)(*[int(r) for r in ubatch_rows])
    (dp,) = _bufs([chunk_done], 4, "chunk_done")
    (tp,) = _bufs([chunk_tiles], 4, "chunk_tiles")
    nf = min(chunk_done.numel(), chunk_tiles.numel())
    _call("ar_reduce_ubatch_flags", _ptr_array(ip), _ptr_array(op), len(ip), int(rows), int(hidden),
          int(n_ubatch), ub, int(chunk_bytes), int(variant), sp, dp, tp, nf, int(epoch) & 0xFFFFFFFF)


def fp8_scale_count(n: int) -> int:
    """Scale bytes per rank for n elements: one per block of 32."""
    return -(-int(n) // FP8_BLOCK)


def ar_quantize_fp8(xs: Sequence, codes: Sequence, scales: Sequence, n: int | None = None,
                    stream=None) -> None:
    """Quantise P bf16 buffers to E4M3 codes (uint8[n]) and per-32-element
    power-of-two scales (uint8[ceil(n/32)], exponent + 127), one launch."""
    n = xs[0].numel() if n is None else int(n)
    xp = _bufs(xs, 2, "xs", n)
    cp = _bufs(codes, 1, "codes", n)
    sp = _bufs(scales, 1, "scales", fp8_scale_count(n))
    if not (len(xp) == len(cp) == len(sp)):
        raise ValueError("need one code and one scale buffer per input")
    _call("ar_quantize_fp8", _ptr_array(xp), _ptr_array(cp), _ptr_array(sp), len(xp), n, _stream(stream))


def ar_reduce_fp8(codes: Sequence, scales: Sequence, outs: Sequence, n: int | None = None,
                  stream=None) -> None:
    """outs[r][:n] = rank-order binary32 sum of the dequantised contributions,
    rounded to bf16; len(outs) is 1 (one share) or P (all-reduce)."""
    n = codes[0].numel() if n is None else int(n)
    cp = _bufs(codes, 1, "codes", n)
    sp = _bufs(scales, 1, "scales", fp8_scale_count(n))
    op = _bufs(outs, 2, "outs", n)
    if len(cp) != len(sp):
        raise ValueError("need one scale buffer per code buffer")
    _call("ar_reduce_fp8", _ptr_array(cp), _ptr_array(sp), len(cp), _ptr_array(op), len(op), n,
          _stream(stream))


def ar_err_init(d_err, stream=None) -> None:
    (ep,) = _bufs([d_err], 8, "d_err", 2)
    _call("ar_err_init", ep, _stream(stream))


def ar_set_launch_shape(kind: int, block: int, vec: int, nt_loads: int, stores: int,
                        wg_per_cu: int) -> None:
    """Set the launch shape of one kernel kind (tuning; process-wide).  `stores`
    is the output store policy: 0 plain, 1 non-temporal, 2 SC1 write-through,
    3 SC1 write-through + non-temporal."""
    _check(lib().ar_set_launch_shape(int(kind), int(block), int(vec), int(nt_loads),
                                     int(stores), int(wg_per_cu)), "ar_set_launch_shape")


def ar_get_launch_shape(kind: int) -> tuple:
    """(block, vec, nt_loads, stores, wg_per_cu) of one kernel kind."""
    v = [ctypes.c_int() for _ in range(5)]
    _check(lib().ar_get_launch_shape(int(kind), *[ctypes.byref(x) for x in v]), "ar_get_launch_shape")
    return tuple(x.value for x in v)


_PREPARABLE = frozenset([ar_reduce_oneshot, ar_reduce_2stage, ar_reduce_2stage_static, ar_pack_fused,
                         ar_unpack_fused, ar_unpack_fused_wait, ar_rd_schedule, ar_reduce_ubatch,
                         ar_reduce_ubatch_flags, ar_quantize_fp8, ar_reduce_fp8, ar_err_init])
