"""Pins of the oracle's fp8-quantised contributions (CPU only).

The reading being pinned: a rank's bf16 buffer travels as E4M3 ("FN")
codes with one power-of-two scale byte per 32-element block, the scale
being the smallest power of two at which no element exceeds 448; the
receiver dequantises exactly and sums in binary32 in rank order, rounding
once to bf16.  Each pin compares the oracle with something it does not
compute itself: PyTorch's float8_e4m3fn conversions (library routines),
closed forms on values that sit on the fp8 grid, the minimality property of
the scale, the rounding error bound, and the already-pinned sequential
bf16 reducer.
"""
import numpy as np
import pytest
import torch

import oracle
from tensor_all_reduce_amd import synth

BLOCK = 32


def bf16_of(values):
    """Exact float32 -> bf16 bits for values that are bf16-representable."""
    f = np.asarray(values, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f), "not bf16-representable"
    return bits


def widen(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def torch_codes(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def dequant(codes, scales):
    vals = np.array([oracle.e4m3_value(c) for c in range(256)], dtype=np.float64)[codes]
    k = scales.astype(np.int64) - 127
    return vals * np.exp2(np.repeat(k, BLOCK)[: codes.size])


# --- E4M3 code values and rounding -------------------------------------------

def test_code_values_match_torch_all_256():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3_value(c) for c in codes], dtype=np.float32)
    both_nan = np.isnan(want) & np.isnan(got)
    assert np.all((want == got) | both_nan)
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_rounding_matches_torch_on_every_bf16_value_in_range():
    f = widen(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    f = f[np.isfinite(f) & (np.abs(f) <= 448)]
    assert np.array_equal(oracle.e4m3_rn_array(f.astype(np.float64)), torch_codes(f))


def test_rounding_matches_torch_on_dense_fp32_ranges():
    # every fp32 pattern around the subnormal/normal boundary and near 448,
    # plus random patterns over the whole range
    lo = np.arange(0x3A000000, 0x3D000000, 7, dtype=np.uint32).view(np.float32)     # 2^-11 .. 2^-5
    hi = np.arange(0x43C00000, 0x43E00001, dtype=np.uint32).view(np.float32)        # 384 .. 448
    rng = np.random.default_rng(11)
    r = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    r = r[np.isfinite(r) & (np.abs(r) <= 448)]
    for f in (lo, -lo, hi, -hi, r):
        assert np.array_equal(oracle.e4m3_rn_array(f.astype(np.float64)), torch_codes(f))


@pytest.mark.parametrize("v,code", [
    (0.0, 0x00), (-0.0, 0x80), (448.0, 0x7E), (-448.0, 0xFE),
    (2.0 ** -10, 0x00),            # half the smallest subnormal: tie, to even (zero)
    (-(2.0 ** -10), 0x80),         # keeps the sign
    (3 * 2.0 ** -11, 0x01),        # above the tie
    (3 * 2.0 ** -10, 0x02),        # tie between codes 1 and 2: even
    (1.0625, 0x38), (1.1875, 0x3A),  # ties in the normal range go to the even mantissa
    (232.0, 0x76), (240.0, 0x77),
    (448.5, 0x7F), (float("inf"), 0x7F), (float("nan"), 0x7F),
])
def test_rounding_hand_cases(v, code):
    assert oracle.e4m3_rn(v) == code


# --- block scale ---------------------------------------------------------------

@pytest.mark.parametrize("j", list(range(-40, 41, 3)) + [119])
def test_scale_at_and_just_above_a_power_of_two_of_448(j):
    at = 448.0 * 2.0 ** j                      # 1.75 * 2^(8+j): bf16-representable up to j = 119
    x = np.zeros(BLOCK, dtype=np.uint16)
    x[5] = bf16_of([at])[0]
    assert oracle.fp8_block_exp(x) == j
    x[5] += 1                                  # the next bf16 value up
    assert oracle.fp8_block_exp(x) == j + 1


def test_scale_special_blocks():
    z = np.zeros(BLOCK, dtype=np.uint16)
    assert oracle.fp8_block_exp(z) == -127                      # all zero
    t = z.copy(); t[0] = 0x0001                                 # smallest subnormal: clamped
    assert oracle.fp8_block_exp(t) == -127
    m = z.copy(); m[3] = 0x7F7F                                 # largest finite bf16
    assert oracle.fp8_block_exp(m) == 120
    s = z.copy(); s[:4] = [0x7FC0, 0x7F80, 0xFF80, 0x3F80]      # NaN and infinities are ignored
    assert oracle.fp8_block_exp(s) == -8                        # 1 <= 448 * 2^-8 = 1.75
    assert oracle.fp8_block_exp(np.array([0x8000, 0xBF80], np.uint16)) == -8   # sign does not matter


def test_scale_is_the_smallest_that_fits():
    rng = np.random.default_rng(5)
    for seed in range(300):
        x = synth.rank_buffers("logmag", 1, BLOCK, 700 + seed)[0]
        x[rng.integers(0, BLOCK)] ^= np.uint16(rng.integers(0, 2) << 15)
        k = oracle.fp8_block_exp(x)
        amax = np.abs(widen(x).astype(np.float64)).max()
        assert amax <= 448.0 * 2.0 ** k
        assert k == -127 or amax > 448.0 * 2.0 ** (k - 1)


# --- quantisation ---------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 31, 32, 33, 95, 4096, 4099])
def test_quant_layout_and_error_bound(n):
    x = synth.rank_buffers("logmag", 1, n, 710 + n)[0]
    codes, scales = oracle.quant_fp8(x)
    assert codes.size == n and scales.size == -(-n // BLOCK)
    for b in range(scales.size):
        assert int(scales[b]) - 127 == oracle.fp8_block_exp(x[b * BLOCK:(b + 1) * BLOCK])
    f = widen(x).astype(np.float64)
    d = dequant(codes, scales)
    k = np.repeat(scales.astype(np.int64) - 127, BLOCK)[:n]
    assert not np.any((codes & 0x7F) == 0x7F)                 # no NaN code for finite input
    normal = np.abs(f) * np.exp2(-k) >= 2.0 ** -6              # scaled input in E4M3's normal range
    err = np.abs(d - f)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(f[normal]))         # half an ulp of 3 bits
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(f), 2.0 ** (k - 10)))
    assert np.array_equal(np.signbit(d), np.signbit(f))


def test_grid_values_round_trip_exactly():
    # integers in [-15, 15] have at most 4 significant bits: on the E4M3 grid
    # for any scale the blocks get, so dequantisation gives them back
    x = synth.integers(5000, -15, 15, 720)
    codes, scales = oracle.quant_fp8(x)
    assert np.array_equal(dequant(codes, scales), widen(x).astype(np.float64))


def test_non_finite_inputs_give_the_nan_code():
    x = np.array([0x3F80, 0x7FC0, 0x7F80, 0xFF80, 0xFFC1, 0x4000] + [0] * 26, dtype=np.uint16)
    codes, scales = oracle.quant_fp8(x)
    assert list(codes[:6]) == [oracle.e4m3_rn(1.0 * 2 ** 7), 0x7F, 0x7F, 0x7F, 0x7F, oracle.e4m3_rn(2.0 * 2 ** 7)]
    assert int(scales[0]) - 127 == -7                          # amax 2 -> 2 <= 448 * 2^-7 = 3.5


def test_quant_matches_torch_after_scaling():
    # with the scale taken from the block exponent, every code is torch's
    # conversion of x / 2^k (x / 2^k is exact in binary32)
    x = np.concatenate([synth.rank_buffers("normal", 1, 8192, 730)[0],
                        synth.rank_buffers("logmag", 1, 8192, 731)[0]])
    codes, scales = oracle.quant_fp8(x)
    k = np.repeat(scales.astype(np.int64) - 127, BLOCK)[: x.size]
    scaled = (widen(x).astype(np.float64) * np.exp2(-k)).astype(np.float32)
    assert np.array_equal(codes, torch_codes(scaled))


# --- reduce ---------------------------------------------------------------------

@pytest.mark.parametrize("P", [1, 2, 3, 5, 8])
def test_reduce_on_grid_integers_is_the_exact_sum(P):
    xs = [synth.integers(3000, -15, 15, 740, p) for p in range(P)]
    q = [oracle.quant_fp8(x) for x in xs]
    got = oracle.reduce_fp8([c for c, _ in q], [s for _, s in q])
    exact = np.sum([widen(x).astype(np.int64) for x in xs], axis=0)
    assert np.array_equal(widen(got), exact.astype(np.float32))


@pytest.mark.parametrize("P,dist", [(2, "normal"), (4, "logmag"), (8, "normal"), (8, "logmag")])
def test_reduce_equals_sequential_bf16_sum_of_dequantised_values(P, dist):
    # every dequantised value of these inputs is bf16-representable, so the
    # fp8 reduce must equal the pinned sequential reducer run on them
    xs = synth.rank_buffers(dist, P, 4099, 750 + P)
    q = [oracle.quant_fp8(x) for x in xs]
    deq = [bf16_of(dequant(c, s).astype(np.float32)) for c, s in q]
    got = oracle.reduce_fp8([c for c, _ in q], [s for _, s in q])
    assert np.array_equal(got, oracle.reduce_seq(deq))


def test_reduce_propagates_non_finite_as_canonical_nan():
    a = np.array([0x3F80, 0x7F80, 0x4000, 0x0000], dtype=np.uint16)
    b = np.array([0x7FC0, 0x3F80, 0xC000, 0x8000], dtype=np.uint16)
    qa, qb = oracle.quant_fp8(a), oracle.quant_fp8(b)
    got = oracle.reduce_fp8([qa[0], qb[0]], [qa[1], qb[1]])
    assert list(got) == [0x7FC0, 0x7FC0, 0x0000, 0x0000]       # 2 + (-2) = +0; +0 + -0 = +0


def test_top_of_the_bf16_range_dequantises_to_infinity():
    # bf16 0x7F78 = 1.9375 * 2^127 and above: k = 120, x / 2^120 >= 248 rounds
    # (ties to even) to 256, and 256 * 2^120 = 2^128 overflows binary32;
    # 0x7F77 stays below the tie and keeps a finite value
    x = np.array([0x7F78, 0x7F7F, 0xFF7A, 0x7F77] + [0] * 28, dtype=np.uint16)
    codes, scales = oracle.quant_fp8(x)
    assert int(scales[0]) - 127 == 120
    assert list(codes[:4]) == [0x78, 0x78, 0xF8, 0x77]       # 256, 256, -256, 240
    got = oracle.reduce_fp8([codes], [scales])
    assert list(got[:4]) == [0x7F80, 0x7F80, 0xFF80, int(bf16_of([240.0 * 2.0 ** 120])[0])]


def test_reduce_empty():
    c = np.zeros(0, dtype=np.uint8)
    s = np.zeros(0, dtype=np.uint8)
    assert oracle.reduce_fp8([c, c], [s, s]).size == 0
