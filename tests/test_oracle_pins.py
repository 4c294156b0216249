"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test names what it pins the oracle to: hand-derived fixtures
(tests/golden/fixtures.json), an exact rational IEEE-754 model
(tests/exact_ieee.py), closed forms on integer data, library routines
(PyTorch's float32 -> bfloat16 conversion, numpy float64 arithmetic),
invariants, and exact counts.  CPU only.
"""
import json
import os

import numpy as np
import pytest
import torch

import exact_ieee as X
import oracle
from tensor_all_reduce_amd import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fixtures.json")))
U64MAX = np.iinfo(np.uint64).max


def h16(s):
    return int(s, 16)


def bits(xs):
    return [np.array([h16(x)], dtype=np.uint16) for x in xs]


def torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- rn (a9)

def test_rn_exhaustive_vs_torch():
    """All 2^32 binary32 patterns: non-NaN results match PyTorch's float32 ->
    bfloat16 conversion bit for bit; every NaN gives 0x7FC0."""
    step = 1 << 24
    base = np.arange(step, dtype=np.uint32)
    u = np.empty(step, dtype=np.uint32)
    got = np.empty(step, dtype=np.uint16)
    ref = torch.empty(step, dtype=torch.bfloat16)
    ref_np = ref.view(torch.int16).numpy().view(np.uint16)
    diff = np.empty(step, dtype=bool)
    nan = np.empty(step, dtype=bool)
    for start in range(0, 1 << 32, step):
        np.add(base, np.uint32(start), out=u)
        f = u.view(np.float32)
        oracle.rn(f, out=got)
        ref.copy_(torch.from_numpy(f))
        np.isnan(f, out=nan)
        np.not_equal(got, ref_np, out=diff)
        diff &= ~nan
        if diff.any():
            i = int(np.argmax(diff))
            raise AssertionError(f"rn mismatch at 0x{int(u[i]):08X}")
        if nan.any():
            assert np.all(got[nan] == 0x7FC0)


def test_rn_ties():
    f = np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x3F808001, 0xBF808000], dtype=np.uint32).view(np.float32)
    assert list(oracle.rn(f)) == [0x3F80, 0x3F82, 0x3F81, 0x3F81, 0xBF80]


# ---------------------------------------------------------------- exact model sanity

def test_exact_model_matches_golden():
    """The independent rational model reproduces every hand-derived value."""
    for c in GOLDEN["reduce"]:
        assert X.seq_sum([h16(x) for x in c["ranks"]]) == h16(c["seq"]), c["name"]
    for c in GOLDEN["rd"]:
        r = [h16(x) for x in c["ranks"]]
        assert X.tree_sum(r, True) == h16(c["r1"]), c["name"]
        assert X.tree_sum(r, False) == h16(c["r2"]), c["name"]
        assert X.seq_sum(r) == h16(c["seq"]), c["name"]


def test_exact_model_decode_encode_roundtrip():
    for b in range(1 << 16):
        v = X.decode_bf16(b)
        if v[0] == "nan":
            assert X.to_bf16(v) == 0x7FC0
        else:
            assert X.to_bf16(v) == b


# ---------------------------------------------------------------- sequential reduce (a2)

@pytest.mark.parametrize("case", GOLDEN["reduce"], ids=lambda c: c["name"])
def test_seq_golden(case):
    got = oracle.reduce_seq(bits(case["ranks"]))
    assert int(got[0]) == h16(case["seq"]), case["why"]


SPECIALS = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80,
                     0x7FC0, 0x7F81, 0xFFC1, 0x3F80, 0xBF80, 0x4B80, 0xCB80, 0x3B80, 0x3380],
                    dtype=np.uint16)


def _mixed_buffers(P, n, seed):
    xs = synth.rank_buffers("normal" if seed % 2 else "logmag", P, n, 900, seed)
    g = np.random.default_rng([901, seed])
    for x in xs:
        k = g.integers(0, max(1, n // 4) + 1)
        idx = g.choice(n, size=k, replace=False)
        x[idx] = g.choice(SPECIALS, size=k)
    return xs


@pytest.mark.parametrize("P", [2, 3, 4, 5, 8])
def test_seq_brute_force_exact_model(P):
    """Random tiny inputs with special values mixed in: the oracle equals the
    exact rational model element by element, bit for bit."""
    for seed in range(12):
        n = 1 + (seed * 7) % 40
        xs = _mixed_buffers(P, n, seed * 10 + P)
        got = oracle.reduce_seq(xs)
        for i in range(n):
            want = X.seq_sum([int(x[i]) for x in xs])
            assert int(got[i]) == want, (P, seed, i, [hex(int(x[i])) for x in xs])


def test_p2_sweep_vs_float64():
    """P=2: every bf16 pattern as rank 0 against 48 rank-1 values.  Reference:
    numpy float64 sum of two bf16 values (exact, or far from any binary32 tie),
    rounded by numpy to binary32 and by PyTorch to bf16; NaN -> 0x7FC0."""
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    rb = np.concatenate([SPECIALS, synth.normal(29, 902)])
    for b in rb:
        bb = np.full(a.size, b, dtype=np.uint16)
        got = oracle.reduce_seq([a, bb])
        fa = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        fb = (bb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        with np.errstate(invalid="ignore", over="ignore"):
            s32 = (fa + fb).astype(np.float32)
        want = torch_bf16_bits(s32).copy()
        want[np.isnan(s32)] = 0x7FC0
        # binary32 x + (-x) = +0 and -0 + -0 = -0: float64 follows the same rule
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"b=0x{int(b):04X} a=0x{int(a[bad[0]]):04X}"


@pytest.mark.parametrize("kind", ["normal", "logmag"])
def test_seq_within_exact_error_bound(kind):
    """|rn(acc) - S| <= 2^-8 (|S| + g) + g + 2^-134 for the exact sum S, with
    g = gamma_{P-1} * sum|x_p| (recursive summation bound)."""
    from fractions import Fraction as F
    P, n = 8, 400
    xs = synth.rank_buffers(kind, P, n, 903)
    got = oracle.reduce_seq(xs)
    u = F(1, 2 ** 24)
    gamma = (P - 1) * u / (1 - (P - 1) * u)
    for i in range(n):
        r = [int(x[i]) for x in xs]
        S = X.exact_sum(r)
        absum = sum(abs(X.value_of(X.decode_bf16(b))) for b in r)
        y = X.value_of(X.decode_bf16(int(got[i])))
        g = gamma * absum
        assert abs(y - S) <= F(1, 256) * (abs(S) + g) + g + F(1, 2 ** 134), (i, r)


@pytest.mark.parametrize("P", [2, 3, 4, 7, 8])
def test_integer_closed_form_all_variants(P):
    """Integers in [-16,16]: every partial sum is exact, so every schedule
    gives the integer sum itself (numpy int64, encoded by the exact model)."""
    n = 6000
    xs = synth.rank_buffers("integers", P, n, 904, P)
    ints = np.stack([(x.astype(np.uint32) << 16).view(np.float32) for x in xs]).astype(np.int64)
    total = ints.sum(axis=0)
    from fractions import Fraction as F
    want = np.array([X.to_bf16(("num", 1 if t < 0 else 0, F(abs(int(t))))) for t in total], dtype=np.uint16)
    assert np.array_equal(oracle.reduce_seq(xs), want)
    for o in oracle.reduce_2stage(xs):
        assert np.array_equal(o, want)
    rows, hidden = 60, 100
    for o in oracle.reduce_ubatch(xs, rows, hidden, 2, None, 1000):
        assert np.array_equal(o, want)
    if P & (P - 1) == 0:
        words = [oracle.pack(x, 5) for x in xs]
        for carry in (False, True):
            outs, err = oracle.rd(words, 5, carry)
            assert int(err[0]) == 0
            for w in outs:
                x, e2 = oracle.unpack(w, 5 + int(np.log2(P)))
                assert int(e2[0]) == 0
                assert np.array_equal(x, want)


def test_special_cases():
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fa = (a.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(fa)
    # x + (+0) = x, except -0 + +0 = +0
    got = oracle.reduce_seq([a, np.zeros_like(a)])
    want = a.copy()
    want[a == 0x8000] = 0
    want[nan] = 0x7FC0
    assert np.array_equal(got, want)
    # x + (-x) = +0 for finite x
    fin = np.isfinite(fa)
    got = oracle.reduce_seq([a, a ^ np.uint16(0x8000)])
    assert np.all(got[fin] == 0)
    assert np.all(got[~fin] == 0x7FC0)
    # P = 2^k equal inputs c: result c * 2^k (exponent + k) unless it overflows
    for k in (1, 2, 3):
        P = 1 << k
        c = synth.normal(2000, 905, k)
        c = c[np.isfinite((c.astype(np.uint32) << 16).view(np.float32))]
        got = oracle.reduce_seq([c] * P)
        want = torch_bf16_bits((c.astype(np.uint32) << 16).view(np.float32) * np.float32(P))
        assert np.array_equal(got, want)
        words = [oracle.pack(c[: c.size // 2 * 2], 0)] * P
        for carry in (False, True):
            outs, _ = oracle.rd(words, 0, carry)
            x, _ = oracle.unpack(outs[0], k)
            assert np.array_equal(x, want[: c.size // 2 * 2])


def test_permutation_within_tolerance():
    """Permuting the ranks moves a result by at most
    max(2^-7 * max(|a|,|b|), 2 gamma_{P-1} sum|x|)."""
    P, n = 8, 20000
    xs = synth.rank_buffers("normal", P, n, 906)
    base = oracle.reduce_seq(xs)
    g = np.random.default_rng(907)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    absum = sum(np.abs(f(x)) for x in xs)
    gamma = (P - 1) * 2.0 ** -24 / (1 - (P - 1) * 2.0 ** -24)
    for _ in range(4):
        perm = g.permutation(P)
        other = oracle.reduce_seq([xs[p] for p in perm])
        a, b = f(base), f(other)
        tol = np.maximum(2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)), 2 * gamma * absum)
        assert np.all(np.abs(a - b) <= tol)
    ints = synth.rank_buffers("integers", P, 5000, 908)
    ref = oracle.reduce_seq(ints)
    assert np.array_equal(ref, oracle.reduce_seq(ints[::-1]))


# ---------------------------------------------------------------- two-stage (a3, a4)

@pytest.mark.parametrize("case", GOLDEN["shard"], ids=lambda c: c["name"])
def test_shard_len_golden(case):
    assert oracle.shard_len(case["P"], case["n"]) == case["S"]


@pytest.mark.parametrize("P,n", [(2, 1), (8, 1), (8, 7), (8, 9), (8, 100), (3, 1000), (8, 4097), (5, 65)])
def test_2stage_invariants(P, n):
    xs = synth.rank_buffers("normal", P, n, 909, n)
    seq = oracle.reduce_seq(xs)
    outs, scratch = oracle.reduce_2stage(xs, return_scratch=True)
    assert np.array_equal(scratch, seq)
    for o in outs:
        assert np.array_equal(o, seq)
    # index-unique check against the exact model on every element
    for i in range(0, n, max(1, n // 64)):
        assert int(outs[-1][i]) == X.seq_sum([int(x[i]) for x in xs])


# ---------------------------------------------------------------- ubatch (a8)

@pytest.mark.parametrize("chunk", [524288, 32768, 2056, 8, 3])
@pytest.mark.parametrize("split", [None, [1, 29], [20, 10]])
def test_ubatch_equals_oneshot(chunk, split):
    P, rows, hidden = 8, 30, 72
    xs = synth.rank_buffers("logmag", P, rows * hidden, 910)
    seq = oracle.reduce_seq(xs)
    outs = oracle.reduce_ubatch(xs, rows, hidden, 2, split, chunk, oracle.TWOSTAGE)
    for o in outs:
        assert np.array_equal(o, seq)
    outs = oracle.reduce_ubatch(xs, rows, hidden, 2, split, chunk, oracle.ONESHOT)
    assert np.array_equal(outs[0], seq)
    for o in outs[1:]:
        assert not o.any()


def test_ubatch_bad_split():
    xs = synth.rank_buffers("normal", 2, 40, 911)
    with pytest.raises(ValueError):
        oracle.reduce_ubatch(xs, 4, 10, 2, [1, 2], 8)


# ---------------------------------------------------------------- pack / unpack (a5, a7)

@pytest.mark.parametrize("case", GOLDEN["pack"], ids=lambda c: c["name"])
def test_pack_golden(case):
    x = np.array([h16(v) for v in case["x"]], dtype=np.uint16)
    w = oracle.pack(x, h16(case["seq"]))
    assert [f"{int(v):016X}" for v in w] == case["words"]


@pytest.mark.parametrize("case", GOLDEN["unpack"], ids=lambda c: c["name"])
def test_unpack_golden(case):
    w = np.array([int(v, 16) for v in case["words"]], dtype=np.uint64)
    x, err = oracle.unpack(w, h16(case["expected"]))
    assert [f"{int(v):04X}" for v in x] == case["x"]
    assert int(err[0]) == case["count"] and int(err[1]) == case["first"]


@pytest.mark.parametrize("seq", [0, 1, 0x7FFFFFFF, 0xFFFFFFFF])
def test_pack_unpack_roundtrip_all_patterns(seq):
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = np.empty(2 * a.size, dtype=np.uint16)
    x[0::2] = a
    x[1::2] = a[::-1]
    w = oracle.pack(x, seq)
    assert np.all((w >> np.uint64(32)) == np.uint64(seq))
    y, err = oracle.unpack(w, seq)
    assert np.array_equal(x, y)
    assert int(err[0]) == 0 and int(err[1]) == U64MAX


def test_unpack_counts_exact():
    x = synth.normal(20000, 912)
    w = oracle.pack(x, 77)
    g = np.random.default_rng(913)
    for k in (1, 5, 333):
        bad = g.choice(w.size, size=k, replace=False)
        wc = w.copy()
        wc[bad] = (wc[bad] & np.uint64(0xFFFFFFFF)) | (np.uint64(78) << np.uint64(32))
        y, err = oracle.unpack(wc, 77)
        assert int(err[0]) == k and int(err[1]) == int(bad.min())
        assert np.array_equal(y, x)
    stale = oracle.pack(x, 76)
    _, err = oracle.unpack(stale, 77)
    assert int(err[0]) == w.size and int(err[1]) == 0
    # counters accumulate across calls; the first index keeps the minimum
    err = oracle.new_err()
    oracle.unpack(stale, 77, err)
    oracle.unpack(w, 77, err)
    assert int(err[0]) == w.size and int(err[1]) == 0


# ---------------------------------------------------------------- recursive doubling (a6)

@pytest.mark.parametrize("case", GOLDEN["rd"], ids=lambda c: c["name"])
def test_rd_golden(case):
    r = [h16(v) for v in case["ranks"]]
    words = [oracle.pack(np.array([b, 0], dtype=np.uint16), 3) for b in r]
    for carry, key in ((False, "r1"), (True, "r2")):
        outs, err = oracle.rd(words, 3, carry)
        assert int(err[0]) == 0
        for w in outs:
            assert int(w[0]) & 0xFFFF == h16(case[key]), (case["name"], key)


@pytest.mark.parametrize("case", GOLDEN["rd_seq"], ids=lambda c: c["name"])
def test_rd_seq_golden(case):
    P, s0 = case["P"], h16(case["seq0"])
    words = [oracle.pack(synth.normal(64, 914, p), s0) for p in range(P)]
    outs, err = oracle.rd(words, s0)
    assert int(err[0]) == 0
    for w in outs:
        assert np.all((w >> np.uint64(32)) == np.uint64(h16(case["out_seq"])))


@pytest.mark.parametrize("P", [2, 4, 8])
def test_rd_vs_exact_tree(P):
    """The per-step partner exchange equals the balanced tree over rank index
    ranges (computed recursively by the exact model), with per-node bf16
    rounding for R1 and binary32 partials for R2; all ranks agree bitwise."""
    for seed in range(6):
        n = 2 * (1 + seed * 5)
        xs = _mixed_buffers(P, n, 915 + seed * 3 + P)
        words = [oracle.pack(x, seed) for x in xs]
        for carry in (False, True):
            outs, err = oracle.rd(words, seed, carry)
            assert int(err[0]) == 0
            first, e = oracle.unpack(outs[0], seed + int(np.log2(P)))
            assert int(e[0]) == 0
            for w in outs[1:]:
                assert np.array_equal(w, outs[0])
            for i in range(n):
                want = X.tree_sum([int(x[i]) for x in xs], round_each_node=not carry)
                assert int(first[i]) == want, (P, seed, carry, i)


def test_rd_p2_equals_seq():
    xs = _mixed_buffers(2, 512, 916)
    seq = oracle.reduce_seq(xs)
    for carry in (False, True):
        outs, _ = oracle.rd([oracle.pack(x, 0) for x in xs], 0, carry)
        x, _ = oracle.unpack(outs[1], 1)
        assert np.array_equal(x, seq)


def test_rd_error_counts_exact():
    P, n = 8, 4000
    xs = synth.rank_buffers("normal", P, n, 917)
    words = [oracle.pack(x, 9) for x in xs]
    W = n // 2
    g = np.random.default_rng(918)
    hits = [(3, 17), (3, 1999), (6, 0), (0, 1500)]
    for r, j in hits:
        words[r][j] = (words[r][j] & np.uint64(0xFFFFFFFF)) | (np.uint64(8) << np.uint64(32))
    outs, err = oracle.rd(words, 9)
    assert int(err[0]) == len(hits)
    assert int(err[1]) == min(r * W + j for r, j in hits)
    # data is still combined from the payload bits
    clean = [oracle.pack(x, 9) for x in xs]
    ref, _ = oracle.rd(clean, 9)
    assert np.array_equal(outs[2], ref[2])
    _ = g


def test_rd_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.rd([oracle.pack(synth.normal(8, 919, p), 0) for p in range(3)], 0)
