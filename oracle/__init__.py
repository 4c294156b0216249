"""CPU oracle of the multi-buffer all-reduce core -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package.  The product path (``tensor_all_reduce_amd``) never
imports, links or calls it; the two share no code.

The arithmetic lives in ``ar_oracle.c`` (plain C, built with gcc, no HIP).
This module only marshals numpy arrays of bf16 bit patterns (``uint16``) and
fused payload words (``uint64``) into it.  Every function follows the
schedule that the C file documents, with the page and section it reads.

Parity pins: every function here is pinned by CPU tests against facts that do
not come from the oracle itself (an exact rational IEEE model, closed forms on
integer data, hand-derived fixtures under ``tests/golden/``, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ar_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = [
    "-O2", "-std=c11", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-Wall", "-Wextra",
]

ONESHOT = 0
TWOSTAGE = 1


def build(verbose: bool = False) -> str:
    """Compile ``ar_oracle.c`` into ``liboracle.so`` with gcc (always rebuilds)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    """Load the oracle library, building it first if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        L.orc_widen.restype = ctypes.c_float
        L.orc_widen.argtypes = [ctypes.c_uint16]
        L.orc_rn.restype = ctypes.c_uint16
        L.orc_rn.argtypes = [ctypes.c_float]
        L.orc_rn_array.restype = None
        L.orc_rn_array.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.orc_reduce_seq.restype = None
        L.orc_reduce_seq.argtypes = [ctypes.c_int, ctypes.POINTER(u16p), ctypes.c_size_t, u16p]
        L.orc_shard_len.restype = ctypes.c_size_t
        L.orc_shard_len.argtypes = [ctypes.c_int, ctypes.c_size_t]
        L.orc_reduce_2stage.restype = ctypes.c_int
        L.orc_reduce_2stage.argtypes = [ctypes.c_int, ctypes.POINTER(u16p), ctypes.c_size_t,
                                        u16p, ctypes.POINTER(u16p)]
        L.orc_reduce_ubatch.restype = ctypes.c_int
        L.orc_reduce_ubatch.argtypes = [ctypes.c_int, ctypes.POINTER(u16p), ctypes.POINTER(u16p),
                                        ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_size_t), ctypes.c_size_t,
                                        ctypes.c_int]
        L.orc_pack.restype = None
        L.orc_pack.argtypes = [u16p, ctypes.c_size_t, ctypes.c_uint32, u64p]
        L.orc_unpack.restype = None
        L.orc_unpack.argtypes = [u64p, ctypes.c_size_t, ctypes.c_uint32, u16p, u64p]
        L.orc_rd.restype = ctypes.c_int
        L.orc_rd.argtypes = [ctypes.c_int, ctypes.POINTER(u64p), ctypes.c_size_t, ctypes.c_uint32,
                             ctypes.c_int, ctypes.POINTER(u64p), u64p]
        u8p = ctypes.POINTER(ctypes.c_uint8)
        L.orc_e4m3_value.restype = ctypes.c_float
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_rn.restype = ctypes.c_uint8
        L.orc_e4m3_rn.argtypes = [ctypes.c_double]
        L.orc_e4m3_rn_array.restype = None
        L.orc_e4m3_rn_array.argtypes = [ctypes.c_void_p, ctypes.c_size_t, u8p]
        L.orc_fp8_block_exp.restype = ctypes.c_int
        L.orc_fp8_block_exp.argtypes = [u16p, ctypes.c_size_t]
        L.orc_quant_fp8.restype = None
        L.orc_quant_fp8.argtypes = [u16p, ctypes.c_size_t, u8p, u8p]
        L.orc_reduce_fp8.restype = ctypes.c_int
        L.orc_reduce_fp8.argtypes = [ctypes.c_int, ctypes.POINTER(u8p), ctypes.POINTER(u8p),
                                     ctypes.c_size_t, u16p]
        _lib = L
    return _lib


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bit patterns, got {a.dtype}")
    return a


def _u64(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint64:
        raise TypeError(f"expected uint64 payload words, got {a.dtype}")
    return a


def _ptr16(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _ptr64(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))


def _ptrs16(arrs):
    T = ctypes.POINTER(ctypes.c_uint16) * len(arrs)
    return T(*[_ptr16(a) for a in arrs])


def _ptrs64(arrs):
    T = ctypes.POINTER(ctypes.c_uint64) * len(arrs)
    return T(*[_ptr64(a) for a in arrs])


def _flat_inputs(xs):
    xs = [_u16(np.asarray(x)).reshape(-1) for x in xs]
    n = xs[0].size
    if any(x.size != n for x in xs):
        raise ValueError("all rank buffers must have the same length")
    return xs, n


def widen(b: int) -> float:
    return float(lib().orc_widen(int(b)))


def rn(values: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """binary32 values -> bf16 bits (nearest, ties to even; NaN -> 0x7FC0)."""
    a = np.ascontiguousarray(values, dtype=np.float32).reshape(-1)
    if out is None:
        out = np.empty(a.size, dtype=np.uint16)
    elif out.dtype != np.uint16 or out.size != a.size or not out.flags.c_contiguous:
        raise ValueError("out must be a contiguous uint16 array of the same size")
    lib().orc_rn_array(a.ctypes.data, a.size, out.ctypes.data)
    return out.reshape(np.shape(values))


def reduce_seq(xs) -> np.ndarray:
    """One-shot: out[i] = rn(((x0 + x1) + x2) + ... + x_{P-1}) in binary32."""
    xs, n = _flat_inputs(xs)
    out = np.empty(n, dtype=np.uint16)
    lib().orc_reduce_seq(len(xs), _ptrs16(xs), n, _ptr16(out))
    return out


def shard_len(P: int, n: int) -> int:
    return int(lib().orc_shard_len(P, n))


def reduce_2stage(xs, return_scratch: bool = False):
    """Two-stage: reduce-scatter into scratch, then all-gather to P outputs."""
    xs, n = _flat_inputs(xs)
    P = len(xs)
    scratch = np.empty(n, dtype=np.uint16)
    outs = [np.empty(n, dtype=np.uint16) for _ in range(P)]
    rc = lib().orc_reduce_2stage(P, _ptrs16(xs), n, _ptr16(scratch), _ptrs16(outs))
    if rc != 0:
        raise MemoryError("oracle two-stage reduce failed")
    return (outs, scratch) if return_scratch else outs


def reduce_ubatch(xs, rows: int, hidden: int, n_ubatch: int = 2, ubatch_rows=None,
                  chunk_elems: int = 524288, variant: int = TWOSTAGE):
    """Chunked multi-ubatch reduce; returns the P outputs (one-shot: only
    outs[0] is written, the others are returned as zeros)."""
    xs, n = _flat_inputs(xs)
    if n != rows * hidden:
        raise ValueError("rows * hidden must equal the buffer length")
    P = len(xs)
    outs = [np.zeros(n, dtype=np.uint16) for _ in range(P)]
    ub = None
    if ubatch_rows is not None:
        ub = (ctypes.c_size_t * n_ubatch)(*[int(r) for r in ubatch_rows])
    rc = lib().orc_reduce_ubatch(P, _ptrs16(xs), _ptrs16(outs), rows, hidden, n_ubatch, ub,
                                 chunk_elems, variant)
    if rc != 0:
        raise ValueError("oracle ubatch reduce: bad split")
    return outs


def pack(x: np.ndarray, seq: int) -> np.ndarray:
    x = _u16(np.asarray(x)).reshape(-1)
    if x.size % 2:
        raise ValueError("pack needs an even element count")
    w = np.empty(x.size // 2, dtype=np.uint64)
    lib().orc_pack(_ptr16(x), x.size, seq & 0xFFFFFFFF, _ptr64(w))
    return w


def new_err() -> np.ndarray:
    return np.array([0, np.iinfo(np.uint64).max], dtype=np.uint64)


def unpack(w: np.ndarray, expected_seq: int, err: np.ndarray | None = None):
    """Returns (x, err) with err = [mismatch count, first bad word index]."""
    w = _u64(np.asarray(w)).reshape(-1)
    err = new_err() if err is None else err
    x = np.empty(w.size * 2, dtype=np.uint16)
    lib().orc_unpack(_ptr64(w), x.size, expected_seq & 0xFFFFFFFF, _ptr16(x), _ptr64(err))
    return x, err


def rd(in_words, seq0: int, fp32_carry: bool = False, err: np.ndarray | None = None):
    """Recursive doubling over P = 2^L payload buffers; returns (outs, err)."""
    ins = [_u64(np.asarray(w)).reshape(-1) for w in in_words]
    P = len(ins)
    W = ins[0].size
    if any(w.size != W for w in ins):
        raise ValueError("all payload buffers must have the same length")
    err = new_err() if err is None else err
    outs = [np.empty(W, dtype=np.uint64) for _ in range(P)]
    rc = lib().orc_rd(P, _ptrs64(ins), 2 * W, seq0 & 0xFFFFFFFF, 1 if fp32_carry else 0,
                      _ptrs64(outs), _ptr64(err))
    if rc != 0:
        raise ValueError("oracle recursive doubling: P must be a power of two in [2, 64]")
    return outs, err


# --- fp8-quantised contributions -------------------------------------------
FP8_BLOCK = 32


def e4m3_value(code: int) -> float:
    """Value of one E4M3 (OCP "FN") code."""
    return float(lib().orc_e4m3_value(int(code) & 0xFF))


def e4m3_rn(v: float) -> int:
    """Nearest E4M3 code to v (|v| <= 448), ties to even; else 0x7F."""
    return int(lib().orc_e4m3_rn(float(v)))


def e4m3_rn_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).reshape(-1)
    out = np.empty(v.size, dtype=np.uint8)
    lib().orc_e4m3_rn_array(v.ctypes.data, v.size, _ptr8(out))
    return out


def fp8_block_exp(x: np.ndarray) -> int:
    x = _u16(np.asarray(x)).reshape(-1)
    return int(lib().orc_fp8_block_exp(_ptr16(x), x.size))


def _ptr8(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def quant_fp8(x: np.ndarray):
    """Returns (codes uint8[n], scales uint8[ceil(n/32)]) for one rank buffer."""
    x = _u16(np.asarray(x)).reshape(-1)
    codes = np.empty(x.size, dtype=np.uint8)
    scales = np.empty(-(-x.size // FP8_BLOCK), dtype=np.uint8)
    lib().orc_quant_fp8(_ptr16(x), x.size, _ptr8(codes), _ptr8(scales))
    return codes, scales


def reduce_fp8(codes, scales) -> np.ndarray:
    """Sum of the dequantised contributions of P ranks, rounded to bf16."""
    cs = [np.ascontiguousarray(c, dtype=np.uint8).reshape(-1) for c in codes]
    ss = [np.ascontiguousarray(s, dtype=np.uint8).reshape(-1) for s in scales]
    n = cs[0].size
    if any(c.size != n for c in cs) or any(s.size != -(-n // FP8_BLOCK) for s in ss) or len(cs) != len(ss):
        raise ValueError("need P code buffers of n bytes and P scale buffers of ceil(n/32) bytes")
    out = np.empty(n, dtype=np.uint16)
    T = ctypes.POINTER(ctypes.c_uint8) * len(cs)
    rc = lib().orc_reduce_fp8(len(cs), T(*[_ptr8(c) for c in cs]), T(*[_ptr8(s) for s in ss]), n,
                              _ptr16(out))
    if rc != 0:
        raise ValueError("oracle fp8 reduce: P must be in [1, 64]")
    return out
