"""Buffers past 2^32 elements: every index computation must be 64-bit.

P = 2 rank buffers of n = 2^32 + 40 bf16 elements (8 GiB each), drawn on
the GPU.  One-shot, fused two-stage, pack -> recursive doubling -> unpack
(16 GiB payload buffers) and the fp8 path run at that size; elements on both
sides of the 2^32 boundary, at the very end, at the start and at random are
compared with the oracle.  Buffers are freed between sections (the largest
section holds about 80 GiB).
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_amd as tar
from tensor_all_reduce_amd import synth
from gpu_util import DEV, note, down16, down64, empty16, bits16, new_err, err_host

pytestmark = pytest.mark.gpu

N = (1 << 32) + 40
P = 2


def sample_idx(n, seed):
    g = np.random.default_rng(seed)
    b = 1 << 32
    idx = np.concatenate([np.arange(0, 256), np.arange(b - 4096, min(n, b + 4096)), np.arange(n - 256, n),
                          np.arange((1 << 31) - 64, (1 << 31) + 64), g.integers(0, n, size=20000)])
    return np.unique(idx)


def gather16(t, idx):
    return down16(bits16(t)[torch.from_numpy(idx.astype(np.int64)).to(DEV)])


def test_past_2_pow_32_elements():
    idx = sample_idx(N, 77)
    note(f"max size: generate 2 x {N} bf16")
    ins = [bits16(t) for t in synth.device_rank_buffers("normal", P, N, 8)]
    xs = [gather16(x, idx) for x in ins]
    ref = oracle.reduce_seq(xs)

    note("max size: oneshot")
    out = empty16(N)
    tar.ar_reduce_oneshot(ins, out)
    torch.cuda.synchronize()
    assert np.array_equal(gather16(out, idx), ref)

    note("max size: 2stage fused")
    out2 = empty16(N)
    tar.ar_reduce_2stage(ins, [out, out2])
    torch.cuda.synchronize()
    assert np.array_equal(gather16(out, idx), ref) and np.array_equal(gather16(out2, idx), ref)
    del out2
    torch.cuda.empty_cache()

    note("max size: fp8 quantise + reduce")
    codes = [torch.empty(N, dtype=torch.uint8, device=DEV) for _ in range(P)]
    scales = [torch.empty(tar.fp8_scale_count(N), dtype=torch.uint8, device=DEV) for _ in range(P)]
    tar.ar_quantize_fp8(ins, codes, scales)
    tar.ar_reduce_fp8(codes, scales, [out])
    torch.cuda.synchronize()
    blocks = np.unique(idx // 32)
    bidx = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    bidx = bidx[bidx < N]
    xb = [gather16(x, bidx) for x in ins]          # the last block is short: n = 2^32 + 40
    q = [oracle.quant_fp8(x) for x in xb]
    tb = torch.from_numpy(bidx.astype(np.int64)).to(DEV)
    for p in range(P):
        assert np.array_equal(codes[p][tb].cpu().numpy(), q[p][0]), f"fp8 codes rank {p}"
        sb = torch.from_numpy(blocks.astype(np.int64)).to(DEV)
        assert np.array_equal(scales[p][sb].cpu().numpy(), q[p][1]), f"fp8 scales rank {p}"
    want = oracle.reduce_fp8([c for c, _ in q], [s for _, s in q])
    assert np.array_equal(gather16(out, bidx), want)
    del codes, scales
    torch.cuda.empty_cache()

    note("max size: pack -> rd -> unpack (16 GiB payloads)")
    W = N // 2
    words = [torch.empty(W, dtype=torch.int64, device=DEV) for _ in range(P)]
    for p in range(P):
        tar.ar_pack_fused(ins[p], words[p], 0xFFFFFFFF)
    rdo = [torch.empty(W, dtype=torch.int64, device=DEV) for _ in range(P)]
    err = new_err()
    tar.ar_rd_schedule(words, rdo, 0xFFFFFFFF, err)
    tar.ar_unpack_fused(rdo[1], out, 0, err)           # seq wraps to 0 after one step
    torch.cuda.synchronize()
    assert err_host(err) == (0, 2 ** 64 - 1)
    widx = np.unique(idx // 2)
    pairs = (widx[:, None] * 2 + np.arange(2)[None, :]).reshape(-1)
    xw = [gather16(x, pairs) for x in ins]
    o_words, o_err = oracle.rd([oracle.pack(x, 0xFFFFFFFF) for x in xw], 0xFFFFFFFF)
    got_w = down64(rdo[0][torch.from_numpy(widx.astype(np.int64)).to(DEV)])
    assert np.array_equal(got_w, o_words[0])
    assert int(o_err[0]) == 0
    want_x, _ = oracle.unpack(o_words[1], 0)
    assert np.array_equal(gather16(out, pairs), want_x)
    del ins, out, words, rdo
    torch.cuda.empty_cache()
