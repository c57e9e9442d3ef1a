"""Pins for the oracle's element/scale codecs: page-printed facts (golden
fixtures), torch's float8 decoders as an independent library, brute force over
the alphabet, and the tie cases of round-to-nearest-even."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split("=", 1)
        out[k.strip()] = v.strip()
    return out


def test_e2m1_alphabet_matches_pages(orc):
    g = _kv("e2m1_alphabet.txt")
    vals = [orc.e2m1_decode(c) for c in range(16)]
    nonneg = sorted({v for v in vals if v >= 0})
    assert nonneg == [float(t) for t in g["nonnegative"].split()]
    assert len(vals) == int(g["codes"])
    # 15 distinct values: +0 and -0 collapse
    assert len({v for v in vals}) == int(g["distinct_values"])
    assert max(vals) == float(g["max"])
    # bit layout S E E M: sign in bit 3, magnitude codes 0..7 ascend
    for c in range(8):
        assert orc.e2m1_decode(c | 8) == -orc.e2m1_decode(c)
        assert math.copysign(1.0, orc.e2m1_decode(c | 8)) == -1.0
    assert [orc.e2m1_decode(c) for c in range(8)] == sorted(nonneg)
    # S E E M: exponent field 0 is subnormal (M * 0.5), 01 -> 1.x, 10 -> 2.x, 11 -> 4.x
    assert orc.e2m1_decode(0b0001) == 0.5
    assert orc.e2m1_decode(0b0010) == 1.0 and orc.e2m1_decode(0b0011) == 1.5
    assert orc.e2m1_decode(0b0100) == 2.0 and orc.e2m1_decode(0b0101) == 3.0
    assert orc.e2m1_decode(0b0110) == 4.0 and orc.e2m1_decode(0b0111) == 6.0


def test_e2m1_homework_closed_form(orc):
    h = _kv("e2m1_homework.txt")
    vals = sorted({orc.e2m1_decode(c) for c in range(16)})
    fr = [Fraction(v) for v in vals]
    assert sum(fr) / len(fr) == Fraction(h["mean"])
    assert sum(v * v for v in fr) == Fraction(h["sum_squares"])
    var = sum((v - sum(fr) / 15) ** 2 for v in fr) / 15
    assert var == Fraction(h["population_std_squared"])


def test_e4m3_decode_all_codes_vs_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([orc.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], ours[~nan])
    # signed zero
    assert math.copysign(1.0, ours[0x80]) == -1.0
    assert ours[0x7E] == 448.0


def test_e8m0_decode_all_codes_vs_torch_and_pages(orc):
    t = _format_table()
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = np.array([orc.e8m0_decode(c) for c in range(256)])
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], ours[:255])
    # pure powers of two, range 2^-127 .. 2^127 (pages)
    for c in range(255):
        m, e = math.frexp(ours[c])
        assert m == 0.5
    assert math.log2(ours[0]) == t["E8M0_MIN_LOG2"]
    assert math.log2(ours[254]) == t["E8M0_MAX_LOG2"]


def _format_table():
    out = {}
    for line in open(os.path.join(GOLDEN, "format_table.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        if len(parts) == 2:
            out[parts[0]] = int(parts[1])
        else:
            out[parts[0]] = tuple(float(p) for p in parts[1:])
    return out


def test_bits_per_element_match_pages(orc):
    t = _format_table()
    for fmt, name in ((orc.MXFP4, "MXFP4"), (orc.NVFP4, "NVFP4"), (orc.MXFP8, "MXFP8")):
        block, sbits, ebits, bpe = t[name]
        rows, cols = 64, 256
        n = rows * cols
        nbytes = orc.tensor_bytes(fmt, rows, cols)
        extra = 32 if fmt == orc.NVFP4 else 0  # one FP32 per tensor ("tiny")
        assert Fraction(8 * nbytes - extra, n) == Fraction(bpe).limit_denominator(64)
        assert orc.scales_bytes(fmt, rows, cols) * block == n
        assert orc.codes_bytes(fmt, rows, cols) * 8 == n * ebits


# --- round-to-nearest-even --------------------------------------------------
E2M1_TIES = [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0)]


@pytest.mark.parametrize("y,want", E2M1_TIES)
def test_e2m1_rne_ties_to_even_code(orc, y, want):
    for s in (1.0, -1.0):
        c = orc.e2m1_encode_rne(s * y)
        assert orc.e2m1_decode(c) == s * want
        # the chosen code of a tie has an even mantissa bit
        assert (c & 1) == 0


def test_e2m1_rne_is_nearest_bruteforce(orc):
    g = np.random.default_rng(1)
    alphabet = np.array([orc.e2m1_decode(c) for c in range(16)])
    ys = np.concatenate([g.uniform(-7, 7, 20000), g.standard_normal(5000) * 1e-3])
    for y in ys.astype(np.float32):
        c = orc.e2m1_encode_rne(float(y))
        v = orc.e2m1_decode(c)
        if abs(y) >= 6:
            assert v == math.copysign(6.0, y)
            continue
        d = np.abs(alphabet - float(y))
        assert abs(v - float(y)) == d.min()
        assert math.copysign(1.0, v) == math.copysign(1.0, float(y))


def test_e4m3_rne_vs_torch_cast(orc):
    g = np.random.default_rng(2)
    ys = np.concatenate([
        g.uniform(-464, 464, 20000),
        g.standard_normal(20000) * 2.0 ** g.integers(-12, 8, 20000),
        # exact midpoints between neighbours, both signs
        [(orc.e4m3_decode(c) + orc.e4m3_decode(c + 1)) / 2 for c in range(0, 126)],
        [-(orc.e4m3_decode(c) + orc.e4m3_decode(c + 1)) / 2 for c in range(0, 126)],
        [464.0, -464.0, 448.0, 2.0 ** -10, 2.0 ** -9, 3 * 2.0 ** -11],
    ]).astype(np.float32)
    ref = torch.from_numpy(ys).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([orc.e4m3_encode_rne(float(y)) for y in ys], np.uint8)
    # torch maps values that round to zero onto +-0 with the input's sign, as we do
    assert np.array_equal(ref, ours)


def test_saturation(orc):
    for y in (6.0, 7.0, 1e30, float("inf")):
        assert orc.e2m1_decode(orc.e2m1_encode_rne(y)) == 6.0
        assert orc.e2m1_decode(orc.e2m1_encode_rne(-y)) == -6.0
        assert orc.e2m1_decode(orc.e2m1_encode_sr(y, 0)) == 6.0
    for y in (448.0, 500.0, 1e30):
        assert orc.e4m3_decode(orc.e4m3_encode_rne(y)) == 448.0
        assert orc.e4m3_decode(orc.e4m3_encode_sr(-y, 12345)) == -448.0


# --- stochastic rounding ----------------------------------------------------
@pytest.mark.parametrize("y", [0.1, 0.3, 0.7, 1.1, 1.3, 2.2, 2.9, 3.3, 4.5, 5.9, -5.1, 2.0 ** -20])
def test_e2m1_sr_exhaustive_count(orc, y):
    """Over all 65536 random values, the number that round up is floor(t),
    t = (|y| - lo) * 2^16 / (hi - lo), and only the two neighbours occur."""
    y = float(np.float32(y))
    a = abs(y)
    vals = sorted({orc.e2m1_decode(c) for c in range(8)})
    lo = max(v for v in vals if v <= a)
    hi = min(v for v in vals if v > a)
    ups = 0
    for r in range(65536):
        v = abs(orc.e2m1_decode(orc.e2m1_encode_sr(y, r)))
        assert v in (lo, hi)
        ups += v == hi
    t = Fraction(a) - Fraction(lo)
    t = t * 65536 / (Fraction(hi) - Fraction(lo))
    assert ups == math.floor(t)


def test_e4m3_sr_exhaustive_count_sampled(orc):
    g = np.random.default_rng(3)
    vals = sorted({orc.e4m3_decode(c) for c in range(127)})
    for y in g.uniform(2.0 ** -9, 440, 6).astype(np.float32):
        a = float(y)
        lo = max(v for v in vals if v <= a)
        hi = min(v for v in vals if v > a)
        rs = np.arange(65536)
        out = np.array([orc.e4m3_decode(orc.e4m3_encode_sr(a, int(r))) for r in rs])
        assert set(np.unique(out)) <= {lo, hi}
        t = (Fraction(a) - Fraction(lo)) * 65536 / (Fraction(hi) - Fraction(lo))
        assert (out == hi).sum() == math.floor(t)
        # the rounding is monotone in r: small r round up
        assert np.all(out[: math.floor(t)] == hi)


def test_sr_unbiased_over_many_draws(orc):
    """The expected value is preserved (pages: "so the expected value is
    preserved"): over N independent Philox draws the mean of the decoded value
    is within 4 sigma / sqrt(N) + (hi - lo) * 2^-16 of y."""
    n = 200000
    for y, enc, dec in ((1.3, orc.e2m1_encode_sr, orc.e2m1_decode),
                        (4.7, orc.e2m1_encode_sr, orc.e2m1_decode),
                        (0.0123, orc.e4m3_encode_sr, orc.e4m3_decode)):
        y = float(np.float32(y))
        s = 0.0
        s2 = 0.0
        for i in range(n):
            v = dec(enc(y, orc.rand16(7, 1000, i)))
            s += v
            s2 += v * v
        mean = s / n
        var = s2 / n - mean * mean
        vals = sorted({abs(dec(c)) for c in range(256 if dec is orc.e4m3_decode else 16)
                       if not math.isnan(dec(c))})
        lo = max(v for v in vals if v <= y)
        hi = min(v for v in vals if v > y)
        bound = 4 * math.sqrt(var / n) + (hi - lo) * 2.0 ** -16
        assert abs(mean - y) <= bound, (y, mean, bound)
