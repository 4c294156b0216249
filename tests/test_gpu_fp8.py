"""fp8-quantised contributions on the GPU (ar_quantize_fp8, ar_reduce_fp8)
against the oracle: codes and scales bit for bit (a floating-point decision
that yields an integer code is taken in binary32 on both sides, on the same
exact quotient x / 2^k), reduced outputs bit for bit (same rank order, same
rounding).  Every call goes through the C-ABI.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_amd as tar
from tensor_all_reduce_amd import synth
from gpu_util import DEV, note, up16, down16, empty16, bits16, sample_indices

pytestmark = pytest.mark.gpu

BLOCK = 32
SENT = 0xA5


def up8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def down8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.uint8)


def code_bufs(P, n, pad=48):
    """Code and scale buffers with a sentinel tail past the end."""
    codes = [torch.full((n + pad,), SENT, dtype=torch.uint8, device=DEV) for _ in range(P)]
    scales = [torch.full((tar.fp8_scale_count(n) + pad,), SENT, dtype=torch.uint8, device=DEV) for _ in range(P)]
    return codes, scales


def gpu_quant(xs_host, pad=48):
    P, n = len(xs_host), xs_host[0].size
    ins = [up16(x) for x in xs_host]
    codes, scales = code_bufs(P, n, pad)
    tar.ar_quantize_fp8(ins, codes, scales, n=n)
    torch.cuda.synchronize()
    return codes, scales


def check_quant(xs_host, codes, scales, what):
    n = xs_host[0].size
    nb = tar.fp8_scale_count(n)
    for p, x in enumerate(xs_host):
        wc, ws = oracle.quant_fp8(x)
        gc, gs = down8(codes[p]), down8(scales[p])
        bad = np.nonzero(gc[:n] != wc)[0]
        assert bad.size == 0, f"{what} rank {p}: {bad.size} code mismatches, first at {bad[0]}: " \
                              f"x={x[bad[0]]:#06x} got {gc[bad[0]]:#04x} want {wc[bad[0]]:#04x}"
        bad = np.nonzero(gs[:nb] != ws)[0]
        assert bad.size == 0, f"{what} rank {p}: {bad.size} scale mismatches, first block {bad[0]}"
        assert np.all(gc[n:] == SENT) and np.all(gs[nb:] == SENT), f"{what} rank {p}: wrote past the end"


@pytest.mark.parametrize("dist", ["normal", "logmag"])
@pytest.mark.parametrize("n", [1, 7, 8, 31, 33, 8192, 3 * 65536 + 37])
def test_quant_matches_oracle(dist, n):
    P = 3
    xs = synth.rank_buffers(dist, P, n, 800, n)
    note(f"fp8 quant {dist} n={n}")
    codes, scales = gpu_quant(xs)
    check_quant(xs, codes, scales, f"{dist} n={n}")


def test_quant_every_bf16_value_at_scale_one():
    """Blocks led by 448 (scale exponent 0) whose other 31 elements sweep every
    finite bf16 pattern of magnitude below 448, both signs: the conversion
    sees every value a contribution can produce (other scales only shift the
    exponent exactly)."""
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (allp.astype(np.uint32) << 16).view(np.float32)
    vals = allp[np.isfinite(f) & (np.abs(f) < 448)]
    nblk = -(-vals.size // 31)
    body = np.zeros(nblk * 31, dtype=np.uint16)
    body[: vals.size] = vals
    x = np.empty(nblk * BLOCK, dtype=np.uint16)
    x.reshape(nblk, BLOCK)[:, 0] = 0x43E0
    x.reshape(nblk, BLOCK)[:, 1:] = body.reshape(nblk, 31)
    note(f"fp8 quant exhaustive, {x.size} elements")
    codes, scales = gpu_quant([x])
    check_quant([x], codes, scales, "exhaustive")
    assert np.all(down8(scales[0])[:nblk] == 127)


def test_quant_scale_edges():
    """Block maxima exactly 448 * 2^j and one bf16 step above, for every j
    whose value is a finite bf16, plus all-zero, subnormal-only, largest-finite
    and non-finite blocks."""
    blocks = []
    for j in range(-140, 120):
        for step in (0, 1):
            v = np.float32(448.0 * 2.0 ** j)
            b = int(v.view(np.uint32) >> 16)
            if not np.isfinite(v) or v == 0 or (b << 16) != int(v.view(np.uint32)):
                continue
            blk = synth.rank_buffers("logmag", 1, BLOCK, 810, j + 200, step)[0] & np.uint16(0x7FFF)
            blk = np.minimum(blk, np.uint16(b))                   # at most the maximum
            blk[(j + 3) % BLOCK] = b + step
            blk[(j + 7) % BLOCK] |= 0x8000
            blocks.append(blk)
    special = [np.zeros(BLOCK, np.uint16),
               np.arange(1, BLOCK + 1, dtype=np.uint16),                    # bf16 subnormals
               np.full(BLOCK, 0x7F7F, np.uint16),                            # largest finite
               np.array([0x7FC0, 0x7F80, 0xFF80, 0xFFC1] + [0x3F80] * 28, np.uint16),
               np.array([0x7F80] * BLOCK, np.uint16),                        # only infinities
               np.array([0x8000] * BLOCK, np.uint16)]                        # only -0
    x = np.concatenate(blocks + special)
    note(f"fp8 quant scale edges, {len(blocks)} + {len(special)} blocks")
    codes, scales = gpu_quant([x])
    check_quant([x], codes, scales, "scale edges")


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("all_out", [False, True])
@pytest.mark.parametrize("n", [16, 4096 + 5, 2 * 65536 + 23])
def test_reduce_matches_oracle(P, all_out, n):
    xs = synth.rank_buffers("logmag" if P % 2 else "normal", P, n, 820, P, n)
    q = [oracle.quant_fp8(x) for x in xs]
    want = oracle.reduce_fp8([c for c, _ in q], [s for _, s in q])
    codes = [up8(c) for c, _ in q]
    scales = [up8(s) for _, s in q]
    nout = P if all_out else 1
    outs = [torch.full((n + 24,), 0x5A5A, dtype=torch.int16, device=DEV) for _ in range(nout)]
    note(f"fp8 reduce P={P} n_out={nout} n={n}")
    tar.ar_reduce_fp8(codes, scales, outs, n=n)
    torch.cuda.synchronize()
    for o in outs:
        g = down16(o)
        bad = np.nonzero(g[:n] != want)[0]
        assert bad.size == 0, f"{bad.size} mismatches, first at {bad[0]}: got {g[bad[0]]:#06x} want {want[bad[0]]:#06x}"
        assert np.all(g[n:] == 0x5A5A)


def test_reduce_every_code_at_several_scales():
    """P = 1: the output is the dequantised value rounded to bf16, for all 256
    codes at scale exponents -127, -20, 0, 7 and 120 (NaN codes give 0x7FC0)."""
    ks = [-127, -20, 0, 7, 120]
    c = np.tile(np.arange(256, dtype=np.uint8), len(ks) * 2)          # 2 blocks of 256 codes per scale
    n = c.size
    s = np.repeat(np.array([k + 127 for k in ks], dtype=np.uint8), 512 // BLOCK)
    want = oracle.reduce_fp8([c], [s])
    out = empty16(n)
    note("fp8 reduce every code")
    tar.ar_reduce_fp8([up8(c)], [up8(s)], [out])
    torch.cuda.synchronize()
    assert np.array_equal(down16(out), want)


@pytest.mark.parametrize("P", [2, 8])
def test_gpu_quant_then_gpu_reduce_end_to_end(P):
    n = 65536 + 40
    xs = synth.rank_buffers("normal", P, n, 830, P)
    q = [oracle.quant_fp8(x) for x in xs]
    want = oracle.reduce_fp8([c for c, _ in q], [s for _, s in q])
    note(f"fp8 end to end P={P}")
    codes, scales = gpu_quant(xs, pad=0)
    outs = [empty16(n) for _ in range(P)]
    tar.ar_reduce_fp8(codes, scales, outs)
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(down16(o), want)


def test_fp8_empty_is_a_no_op():
    x = up16(np.zeros(8, np.uint16))
    c = torch.full((16,), SENT, dtype=torch.uint8, device=DEV)
    s = torch.full((16,), SENT, dtype=torch.uint8, device=DEV)
    out = torch.full((8,), 0x1234, dtype=torch.int16, device=DEV)
    tar.ar_quantize_fp8([x], [c], [s], n=0)
    tar.ar_reduce_fp8([c], [s], [out], n=0)
    torch.cuda.synchronize()
    assert np.all(down8(c) == SENT) and np.all(down8(s) == SENT) and np.all(down16(out) == 0x1234)


def test_fp8_full_size_prefill():
    """P = 8, [16384 x 8192] per rank, N(0,1): quantise all 8 buffers in one
    launch, reduce into all 8 outputs.  Sampled whole blocks of codes and
    scales, and sampled outputs, against the oracle; all outputs identical."""
    P, n = 8, 16384 * 8192
    note("fp8 full size: generate")
    ins = [bits16(t) for t in synth.device_rank_buffers("normal", P, n, 6)]
    codes = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(P)]
    scales = [torch.empty(tar.fp8_scale_count(n), dtype=torch.uint8, device=DEV) for _ in range(P)]
    note("fp8 full size: quantise")
    tar.ar_quantize_fp8(ins, codes, scales)
    outs = [empty16(n) for _ in range(P)]
    note("fp8 full size: reduce")
    tar.ar_reduce_fp8(codes, scales, outs)
    torch.cuda.synchronize()
    blocks = np.unique(sample_indices(n, 20000, 61) // BLOCK)
    idx = (blocks[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    ti = torch.from_numpy(idx.astype(np.int64)).to(DEV)
    tb = torch.from_numpy(blocks.astype(np.int64)).to(DEV)
    xs = [down16(x[ti]) for x in ins]
    q = [oracle.quant_fp8(x) for x in xs]               # sampled blocks are whole blocks
    for p in range(P):
        assert np.array_equal(down8(codes[p][ti]), q[p][0]), f"rank {p} codes"
        assert np.array_equal(down8(scales[p][tb]), q[p][1]), f"rank {p} scales"
    want = oracle.reduce_fp8([c for c, _ in q], [s for _, s in q])
    assert np.array_equal(down16(outs[0][ti]), want)
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    del ins, codes, scales, outs
    torch.cuda.empty_cache()
