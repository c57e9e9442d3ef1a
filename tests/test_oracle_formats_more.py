"""Pins for the oracle's other MX element types: FP8 E5M2, FP6 E3M2 and E2M3,
and INT8 (two's complement with 6 fraction bits -- also the reading of the
block-scaled "S2F6" combine format).

Each decoder is tied to an independent routine or to an already pinned one:
E5M2 to torch's float8_e5m2; every normal E2M3 value to torch's E4M3 and its
codes with the low mantissa bits clear to the pinned E2M1 decoder; every E3M2
value to torch's E5M2; INT8 rounding to numpy's round-half-even.  The FP6
packing reading is pinned by a hand-worked row."""
import math

import numpy as np
import pytest
import torch


def _torch_decode(dtype, n=256):
    return torch.arange(n, dtype=torch.uint8).view(dtype).float().numpy().astype(np.float64)


def _pos_alphabet(orc, fmt, ncodes, sign_bit):
    vals = {orc.elem_decode(fmt, c) for c in range(ncodes) if not c & sign_bit}
    return sorted(v for v in vals if math.isfinite(v))


def test_e5m2_decode_equals_torch(orc):
    want = _torch_decode(torch.float8_e5m2)
    got = np.array([orc.elem_decode(orc.MXFP8_E5M2, c) for c in range(256)])
    both_nan = np.isnan(want) & np.isnan(got)
    assert np.array_equal(got[~both_nan], want[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert orc.elem_decode(orc.MXFP8_E5M2, 0x7B) == 57344.0


def test_e5m2_rne_encode_equals_torch_in_range(orc):
    g = np.random.default_rng(2)
    y = np.concatenate([g.standard_normal(4000) * np.exp(g.uniform(-14, 10, 4000)),
                        [0.0, -0.0, 57344.0, -57344.0, 2.0**-16, 1.5 * 2.0**-16]])
    y = y.astype(np.float32)
    want = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = np.array([orc.elem_encode_rne(orc.MXFP8_E5M2, float(v)) for v in y], np.uint8)
    assert np.array_equal(got, want)
    # beyond the largest finite value the encoder saturates (torch would give Inf)
    assert orc.elem_encode_rne(orc.MXFP8_E5M2, 1e6) == 0x7B
    assert orc.elem_encode_rne(orc.MXFP8_E5M2, -1e6) == 0xFB


def test_e2m3_against_e4m3_and_e2m1(orc):
    """Normal E2M3 values are exactly the E4M3 values in [1, 7.5]; its codes
    with both low mantissa bits clear decode as the E2M1 code c >> 2; the
    subnormal step is 1/8; 32 distinct magnitudes, no NaN or Inf."""
    pos = _pos_alphabet(orc, orc.MXFP6_E2M3, 64, 0x20)
    e4 = _torch_decode(torch.float8_e4m3fn)
    normal = sorted({v for v in e4 if 1.0 <= v <= 7.5})
    assert [v for v in pos if v >= 1.0] == normal
    assert [v for v in pos if v < 1.0] == [k / 8 for k in range(8)]
    assert len(pos) == 32
    for c in range(64):
        if c & 3 == 0:
            assert orc.elem_decode(orc.MXFP6_E2M3, c) == orc.e2m1_decode(c >> 2)
        assert math.isfinite(orc.elem_decode(orc.MXFP6_E2M3, c))


def test_e3m2_against_e5m2(orc):
    """Every E3M2 value is an E5M2 value: the normal ones are the E5M2 values
    in [1/4, 28] (code (e + 12, m) of E5M2), the subnormals are 1/16, 2/16,
    3/16; no NaN or Inf."""
    pos = _pos_alphabet(orc, orc.MXFP6_E3M2, 64, 0x20)
    e5 = _torch_decode(torch.float8_e5m2)
    normal = sorted({v for v in e5 if 0.25 <= v <= 28.0})
    assert [v for v in pos if v >= 0.25] == normal
    assert [v for v in pos if v < 0.25] == [0.0, 1 / 16, 2 / 16, 3 / 16]
    e5codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).float().numpy()
    for c in range(64):
        e, m = (c >> 2) & 7, c & 3
        v = orc.elem_decode(orc.MXFP6_E3M2, c)
        assert math.isfinite(v)
        if e:
            assert v == (-1 if c & 0x20 else 1) * float(e5codes[((e + 12) << 2) | m])


def test_fp6_rne_and_sr_follow_the_shared_rules(orc):
    """Nearest value, ties to the even code, saturation; SR's count of random
    values that round up is floor(t) exactly (the rule pinned for E2M1/E4M3)."""
    for fmt, sign in ((orc.MXFP6_E3M2, 0x20), (orc.MXFP6_E2M3, 0x20)):
        pos = _pos_alphabet(orc, fmt, 64, sign)
        for lo, hi in zip(pos[:-1], pos[1:]):
            mid = 0.5 * (lo + hi)
            c = orc.elem_encode_rne(fmt, mid)
            assert orc.elem_decode(fmt, c) in (lo, hi) and c % 2 == 0
            assert orc.elem_decode(fmt, orc.elem_encode_rne(fmt, lo + 0.3 * (hi - lo))) == lo
            assert orc.elem_decode(fmt, orc.elem_encode_rne(fmt, -(lo + 0.7 * (hi - lo)))) == -hi
        assert orc.elem_decode(fmt, orc.elem_encode_rne(fmt, 1e9)) == pos[-1]
        lo, hi = pos[10], pos[11]
        y = lo + 0.375 * (hi - lo)
        ups = sum(orc.elem_decode(fmt, orc.elem_encode_sr(fmt, y, r)) == hi for r in range(0, 65536, 1))
        assert ups == int(0.375 * 65536)


def test_int8_rne_equals_numpy_rint(orc):
    g = np.random.default_rng(5)
    y = np.concatenate([g.uniform(-2.2, 2.2, 3000), np.arange(-260, 260) / 128.0])
    got = np.array([orc.elem_encode_rne(orc.MXINT8, float(v)) for v in y], np.uint8)
    want = np.clip(np.rint(y * 64), -128, 127).astype(np.int64).astype(np.int8).view(np.uint8)
    assert np.array_equal(got, want)
    assert orc.elem_decode(orc.MXINT8, 0x80) == -2.0 and orc.elem_decode(orc.MXINT8, 0x7F) == 127 / 64
    assert orc.elem_encode_rne(orc.MXINT8, -0.0) == 0


@pytest.mark.parametrize("y", [0.3 / 64 + 5 / 64, -(0.3 / 64 + 5 / 64), -1.5 + 0.8 / 64])
def test_int8_sr_rounds_toward_plus_infinity_with_probability_t(orc, y):
    """Fixed-point SR acts on the signed value: with lo <= y < lo + 1/64, the
    number of 16-bit values that give lo + 1/64 is floor((y - lo) * 64 * 2^16)."""
    lo = math.floor(y * 64) / 64
    t = math.floor((y - lo) * 64 * 65536)
    ups = sum(orc.elem_decode(orc.MXINT8, orc.elem_encode_sr(orc.MXINT8, y, r)) == lo + 1 / 64
              for r in range(65536))
    assert ups == t


def test_fp6_packing_worked_row(orc):
    """READING of the FP6 packing: element c at bits 6c .. 6c+5 of the row's
    little-endian bit string.  Codes 1, 2, 3, 4 give the 24-bit word
    1 + (2 << 6) + (3 << 12) + (4 << 18) = 0x103081: bytes 81 30 10."""
    vals = [orc.elem_decode(orc.MXFP6_E2M3, c) for c in (1, 2, 3, 4)]  # 1/8 .. 4/8
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = vals
    x[0, 31] = 7.5  # block max 7.5: the scale is 2^0 (emax 2, floor(log2 7.5) = 2)
    codes, scales, _ = orc.quantize(x, orc.MXFP6_E2M3)
    assert scales[0, 0] == 127
    assert codes.shape == (1, 24)
    assert list(codes[0, :3]) == [0x81, 0x30, 0x10]
    assert codes[0, 21:].tobytes() == bytes([0, 0, 0x7C])  # element 31 = code 0x1F << 2 in the top byte


@pytest.mark.parametrize("fmt,emax", [(4, 0), (5, 15), (6, 4), (7, 2)])
def test_scale_rule_for_the_other_elements(orc, fmt, emax):
    """A block whose max is 2^k gets scale code k - emax + 127 and its max
    encodes exactly to 2^emax; dequantization returns power-of-two blocks
    exactly."""
    for k in (-90, -3, 0, 5, 60):
        x = np.zeros((1, 32), np.float32)
        x[0, 7] = 2.0 ** k
        x[0, 8] = -(2.0 ** (k - 1))
        codes, scales, _ = orc.quantize(x, fmt)
        assert scales[0, 0] == k - emax + 127
        y = orc.dequantize(fmt, codes, scales, None, 1, 32)
        assert y[0, 7] == 2.0 ** k and y[0, 8] == -(2.0 ** (k - 1))


def test_s2f6_codec_round_trip_is_exact_on_representable_values(orc):
    """RHT16 then block-scaled INT8 (the combine codec), then decode and the
    inverse transform: if the transformed values are multiples of 2^-6 below
    2 with a block maximum of at least 1, every step is exact and x comes
    back bit for bit."""
    g = np.random.default_rng(3)
    mask = orc.rht_signs(9)
    k = g.integers(-127, 128, (8, 256))
    k[:, ::32] = 100  # each block's max >= 1, so its scale is 2^0
    y = (k / 64.0).astype(np.float32)
    x = orc.rht16(y, mask, inverse=True)
    codes, scales, _ = orc.quantize(x, orc.MXINT8, rht=True, sign_mask=mask)
    assert np.all(scales == 127)
    assert np.array_equal(codes.view(np.int8).astype(np.int64), k)
    back = orc.rht16(orc.dequantize(orc.MXINT8, codes, scales, None, 8, 256), mask, inverse=True)
    assert np.array_equal(back, x)
