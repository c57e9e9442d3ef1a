"""Pins for the oracle's quantizers, Hadamard transform, decoder and
requant-transpose: closed forms, invariants and brute force on small inputs."""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads as W


def f32_to_bits(x):
    return np.ascontiguousarray(x, np.float32)


def _grid(orc, fmt):
    if fmt == orc.MXFP8:
        v = [orc.e4m3_decode(c) for c in range(256)]
    else:
        v = [orc.e2m1_decode(c) for c in range(16)]
    return np.array(sorted({x for x in v if not math.isnan(x)}))


def _elem(orc, fmt, codes, r, c):
    if fmt == orc.MXFP8:
        return orc.e4m3_decode(int(codes[r, c]))
    b = int(codes[r, c // 2])
    return orc.e2m1_decode((b >> 4) if c & 1 else (b & 0xF))


# --- MX scale rule ----------------------------------------------------------
@pytest.mark.parametrize("fmt,emax", [(1, 8), (2, 2)])
def test_mx_scale_closed_form_power_of_two_max(orc, fmt, emax):
    """A block whose max is m * 2^k (m in [1,2)) gets scale code k - emax + 127;
    a power-of-two maximum lands exactly on 2^emax after scaling."""
    for k in (-100, -20, -1, 0, 1, 7, 60):
        for m in (1.0, 1.5, 1.9921875):
            x = np.zeros((1, 32), np.float32)
            x[0, 5] = m * 2.0 ** k
            x[0, 6] = -0.25 * 2.0 ** k
            codes, scales, _ = orc.quantize(x, fmt)
            assert scales[0, 0] == k - emax + 127
            if m == 1.0:
                assert _elem(orc, fmt, codes, 0, 5) == 2.0 ** emax


@pytest.mark.parametrize("fmt", [1, 2])
def test_mx_scaled_block_max_invariant(orc, fmt):
    """Unless clamped, the scaled block max lies in [2^emax, 2^(emax+1)); the
    scale code equals floor(log2 amax) - emax + 127, found here by integer
    exponent extraction from the FP32 bits (a different route from frexp)."""
    emax = 8 if fmt == orc.MXFP8 else 2
    g = np.random.default_rng(5)
    x = (g.standard_normal((64, 256)) * np.exp(g.uniform(-20, 20, (64, 1)))).astype(np.float32)
    codes, scales, _ = orc.quantize(x, fmt)
    blocks = np.abs(x).reshape(64, 8, 32).max(axis=2)
    bits = blocks.view(np.uint32)
    expo = ((bits >> 23) & 0xFF).astype(np.int64) - 127
    assert np.array_equal(scales.astype(np.int64), expo - emax + 127)
    scaled = blocks.astype(np.float64) * 2.0 ** -(scales.astype(np.float64) - 127)
    assert np.all((scaled >= 2.0 ** emax) & (scaled < 2.0 ** (emax + 1)))


@pytest.mark.parametrize("fmt", [1, 2])
def test_mx_rne_elements_are_nearest_in_block_grid(orc, fmt):
    """Brute force: each decoded element is the nearest point of the block's
    grid X * alphabet to x (saturating beyond the largest)."""
    g = np.random.default_rng(6)
    x = (g.standard_normal((8, 64)) * 3).astype(np.float32)
    x[0, 3] = 1000.0
    codes, scales, _ = orc.quantize(x, fmt)
    grid = _grid(orc, fmt)
    for r in range(8):
        for c in range(64):
            X = 2.0 ** (int(scales[r, c // 32]) - 127)
            v = _elem(orc, fmt, codes, r, c) * X
            cand = grid * X
            best = np.abs(cand - float(x[r, c])).min()
            assert abs(v - float(x[r, c])) == best


def test_mx_zero_block_and_nan_block(orc):
    x = np.zeros((2, 64), np.float32)
    x[0, 1] = -0.0
    x[1, 40] = np.nan
    x[1, 0] = 3.0
    for fmt in (orc.MXFP8, orc.MXFP4):
        codes, scales, _ = orc.quantize(x, fmt)
        assert scales[0, 0] == 0 and scales[0, 1] == 0  # all-zero blocks: 2^-127
        assert scales[1, 1] == 0xFF  # NaN block
        if fmt == orc.MXFP8:
            assert codes[0, 1] == 0x80  # -0 keeps its sign
            assert np.all(codes[1, 32:] == 0)
        else:
            assert codes[0, 0] == 0x80  # element 1 (high nibble) is -0
            assert np.all(codes[1, 16:] == 0)


def test_mx_bf16_input_equals_f32_input(orc):
    A = W.normal_bf16(16, 64, seed=1, tensor_id=1)
    f = W.bf16_bits_to_f32(A)
    for fmt in (orc.MXFP8, orc.MXFP4):
        a = orc.quantize(A, fmt)
        b = orc.quantize(np.ascontiguousarray(f), fmt)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_mx_exactly_representable_roundtrip(orc):
    """Values already on the block grid survive quantize -> dequantize exactly."""
    g = np.random.default_rng(8)
    for fmt in (orc.MXFP8, orc.MXFP4):
        grid = _grid(orc, fmt)
        x = g.choice(grid, size=(4, 64)).astype(np.float64)
        x[:, 0] = grid.max()  # pin the block maximum so the scale is 2^0
        x[:, 32] = grid.max()
        x = (x * 2.0 ** 3).astype(np.float32)
        codes, scales, _ = orc.quantize(x, fmt)
        y = orc.dequantize(fmt, codes, scales, None, 4, 64)
        assert np.array_equal(y, x)


def test_mx_sr_uses_output_index_stream(orc):
    """SR draws the random value of element n from the stream position n of the
    output: changing the counter by 1 shifts the stream by 8 elements."""
    x = (np.random.default_rng(9).standard_normal((4, 64)) * 0.7).astype(np.float32)
    c0 = orc.quantize(x, orc.MXFP8, orc.SR, seed=3, counter=10)[0]
    # element-wise re-derivation from the scalar SR encoder
    _, scales, _ = orc.quantize(x, orc.MXFP8, orc.RNE)
    for r in range(4):
        for c in range(64):
            X = 2.0 ** (int(scales[r, c // 32]) - 127)
            y = float(x[r, c]) / X
            want = orc.e4m3_encode_sr(y, orc.rand16(3, 10, r * 64 + c))
            assert c0[r, c] == want


# --- NVFP4 -----------------------------------------------------------------
def test_nvfp4_tensor_scale_and_max_block(orc):
    g = np.random.default_rng(10)
    x = (g.standard_normal((16, 64)) * 5).astype(np.float32)
    codes, scales, S = orc.quantize(x, orc.NVFP4)
    T = float(np.abs(x).max())
    assert S == float(np.float32(T) / np.float32(2688.0))
    # S * 2688 recovers T to within one FP32 ulp
    assert abs(S * 2688.0 - T) <= float(np.spacing(np.float32(T)))
    # the block holding T gets the largest E4M3 scale, 448 (code 0x7E)
    r, c = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert scales[r, c // 16] == 0x7E
    # storage: 4.5 bits per element + one FP32 per tensor
    assert codes.nbytes + scales.nbytes == x.size * 4.5 / 8


def test_nvfp4_elements_nearest_to_scaled_value(orc):
    """Brute force: each element code is the nearest E2M1 value to the FP32
    y = x * (1 / (e4m3 * S)) of the pages' two-level decode x ~ e2m1*e4m3*S."""
    g = np.random.default_rng(12)
    x = (g.standard_normal((8, 64)) * np.exp(g.uniform(-3, 3, (8, 1)))).astype(np.float32)
    codes, scales, S = orc.quantize(x, orc.NVFP4)
    alpha = np.array([orc.e2m1_decode(c) for c in range(16)])
    S32 = np.float32(S)
    for r in range(8):
        for c in range(64):
            sb = orc.e4m3_decode(int(scales[r, c // 16]))
            rcp = np.float32(1.0) / (np.float32(sb) * S32)
            y = float(np.float32(x[r, c]) * rcp)
            b = int(codes[r, c // 2])
            v = orc.e2m1_decode((b >> 4) if c & 1 else (b & 0xF))
            if abs(y) >= 6:
                assert v == math.copysign(6.0, y)
            else:
                assert abs(v - y) == np.abs(alpha - y).min()
    # block scales: nearest E4M3 to amax / (6 S), computed in FP32
    e4 = np.array([orc.e4m3_decode(c) for c in range(127)])
    amax = np.abs(x).reshape(8, 4, 16).max(axis=2)
    for r in range(8):
        for b in range(4):
            q = float(np.float32(amax[r, b]) / (np.float32(6.0) * S32))
            got = orc.e4m3_decode(int(scales[r, b]))
            assert abs(got - q) == np.abs(e4 - q).min()


def test_nvfp4_zero_tensor_and_amax_override(orc):
    x = np.zeros((2, 32), np.float32)
    x[1, 3] = -0.0
    codes, scales, S = orc.quantize(x, orc.NVFP4)
    assert S == 1.0 and np.all(scales == 0)
    assert codes[1, 1] == 0x80  # element 3 -> high nibble of byte 1, -0
    y = np.ones((2, 32), np.float32)
    c1, s1, S1 = orc.quantize(y, orc.NVFP4, amax=2.0)
    assert S1 == float(np.float32(2.0) / np.float32(2688.0))


def test_nvfp4_tiny_tensor_scale_overflowing_reciprocal(orc):
    """T = 1.75 * 2^-126 gives S ~ 2^-136.6, so a block whose scale decodes
    to the smallest E4M3 value has 1 / (e4m3 * S) = +Inf in FP32.  Its nonzero
    elements become +-Inf and saturate to +-6 (codes 7 / 0xF), and its zero
    elements keep +-0 (codes 0 / 8) under both roundings."""
    T = np.float32(1.75) * np.float32(2.0) ** -126
    S = np.float32(T) / np.float32(2688.0)
    assert np.isinf(np.float32(1.0) / (np.float32(2.0 ** -9) * S))
    x = np.zeros((1, 32), np.float32)
    # block 0: maximum near 2^-9 * 6 S, so its scale code is 1 (2^-9)
    m = np.float32(6.0 * 2.0 ** -9) * S
    x[0, 0:4] = [m, -m, np.float32(0.0), np.float32(-0.0)]
    x[0, 4] = np.float32(m * 0.25)
    x[0, 16] = T  # block 1 holds the amax
    for rnd in (orc.RNE, orc.SR):
        codes, scales, S_out = orc.quantize(x, orc.NVFP4, rnd, seed=1, amax=float(T))
        assert S_out == float(S)
        assert scales[0, 0] == 1
        nib = [(int(codes[0, c // 2]) >> (4 * (c & 1))) & 0xF for c in range(16)]
        assert nib[0] == 0x7 and nib[1] == 0xF and nib[4] == 0x7  # +-Inf saturates
        assert nib[2] == 0x0 and nib[3] == 0x8  # signed zeros
        assert all(n in (0x0, 0x8) for n in nib[5:])  # the other zeros


def test_nvfp4_dequant_single_rounding(orc):
    g = np.random.default_rng(13)
    x = g.standard_normal((4, 32)).astype(np.float32)
    codes, scales, S = orc.quantize(x, orc.NVFP4)
    y = orc.dequantize(orc.NVFP4, codes, scales, S, 4, 32)
    e = orc.dequantize_f64(orc.NVFP4, codes, scales, 4, 32)
    assert np.array_equal(y, (e.astype(np.float32) * np.float32(S)))
    assert np.array_equal(e.astype(np.float32).astype(np.float64), e)  # product is exact in FP32


def test_nvfp4_sr_unbiased_blockwise(orc):
    """Averaged over many seeds, SR decodes to the FP32 scaled input within the
    SR bias bound (expected value preserved)."""
    x = np.array([[0.3, 1.7, -2.2, 5.3, 0.01, 3.9, -4.4, 1.1] * 2], np.float32)
    _, scales, S = orc.quantize(x, orc.NVFP4)
    n = 4000
    acc = np.zeros(16)
    for s in range(n):
        codes, sc, S2 = orc.quantize(x, orc.NVFP4, orc.SR, seed=s)
        assert np.array_equal(sc, scales) and S2 == S
        acc += orc.dequantize_f64(orc.NVFP4, codes, sc, 1, 16)[0]
    mean = acc / n
    sb = orc.e4m3_decode(int(scales[0, 0]))
    rcp = np.float32(1.0) / (np.float32(sb) * np.float32(S))
    y = (x[0] * rcp).astype(np.float64) * sb
    assert np.all(np.abs(mean - y) <= 4 * 2.0 * sb / np.sqrt(n) + 2.0 * sb * 2.0 ** -16)


# --- Hadamard transform -----------------------------------------------------
def _H16():
    H = np.ones((16, 16))
    for i in range(16):
        for j in range(16):
            H[i, j] = -1.0 if bin(i & j).count("1") % 2 else 1.0
    return H


def test_rht16_one_hot_columns(orc):
    H = _H16()
    for mask in (0, 0xFFFF, 0xA5C3):
        for k in range(16):
            x = np.zeros((1, 16), np.float32)
            x[0, k] = 1.0
            y = orc.rht16(x, mask)[0]
            sgn = -1.0 if (mask >> k) & 1 else 1.0
            assert np.array_equal(y, (0.25 * sgn * H[:, k]).astype(np.float32))


def test_rht16_matches_explicit_matrix_and_is_orthonormal(orc):
    H = _H16()
    g = np.random.default_rng(14)
    x = g.standard_normal((32, 64)).astype(np.float32)
    mask = 0x3C96
    D = np.diag([-1.0 if (mask >> j) & 1 else 1.0 for j in range(16)])
    Mx = 0.25 * H @ D
    y = orc.rht16(x, mask).astype(np.float64)
    ref = (x.astype(np.float64).reshape(32, 4, 16) @ Mx.T).reshape(32, 64)
    # four FP32 butterfly roundings on sums of at most 16 terms
    bound = 4 * 2.0 ** -24 * (np.abs(x).reshape(32, 4, 16).sum(axis=2) * 0.25 * 2)
    assert np.all(np.abs(y - ref).reshape(32, 4, 16) <= bound[..., None] + 1e-30)
    # norm preserved (orthonormal) to FP32 accuracy
    n0 = np.linalg.norm(x.reshape(-1, 16).astype(np.float64), axis=1)
    n1 = np.linalg.norm(y.reshape(-1, 16), axis=1)
    assert np.allclose(n0, n1, rtol=1e-6)


def test_rht16_inverse_is_exact_on_small_integers(orc):
    g = np.random.default_rng(15)
    x = g.integers(-100, 100, (8, 64)).astype(np.float32)
    for mask in (0, 0x1234, 0xFFFF):
        y = orc.rht16(x, mask)
        z = orc.rht16(y, mask, inverse=True)
        assert np.array_equal(z, x)


def test_rht_feeds_quantizer_in_fp32(orc):
    A = W.normal_bf16(8, 64, seed=2, tensor_id=3)
    mask = orc.rht_signs(0)
    y = orc.rht16(A, mask)
    for fmt in (orc.MXFP8, orc.MXFP4, orc.NVFP4):
        a = orc.quantize(A, fmt, rht=True, sign_mask=mask)
        b = orc.quantize(y, fmt)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]
    assert orc.tensor_amax(A, rht=True, sign_mask=mask) == float(np.abs(y).max())


# --- requant-transpose ------------------------------------------------------
def test_requant_transpose_is_dequant_transpose_quantize(orc):
    X = W.normal_bf16(64, 48, seed=3, tensor_id=4, outlier_entries=0.01, outlier_mult=30)
    nv = orc.quantize(X, orc.NVFP4)
    xhat = orc.dequantize(orc.NVFP4, nv[0], nv[1], nv[2], 64, 48)
    for rnd in (orc.RNE, orc.SR):
        codes, scales = orc.requant_transpose(64, 48, rnd, seed=5, counter=17, nvfp4=nv)
        want = orc.quantize(np.ascontiguousarray(xhat.T), orc.MXFP8, rnd, seed=5, counter=17)
        assert codes.shape == (48, 64) and scales.shape == (48, 2)
        assert np.array_equal(codes, want[0]) and np.array_equal(scales, want[1])


def test_requant_transpose_bf16_source(orc):
    dY = W.normal_bf16(64, 32, seed=4, tensor_id=5)
    codes, scales = orc.requant_transpose(64, 32, orc.SR, seed=1, counter=3, bf16=dY)
    want = orc.quantize(np.ascontiguousarray(dY.T), orc.MXFP8, orc.SR, seed=1, counter=3)
    assert np.array_equal(codes, want[0]) and np.array_equal(scales, want[1])


# --- round-trip error statistics ---------------------------------------------
def test_roundtrip_stats_closed_forms(orc):
    """Closed forms: y = x gives zeros; y = x + c gives n c^2, n c, |c|;
    sum x^2 is the plain sum of squares."""
    g = np.random.default_rng(3)
    x = g.standard_normal((16, 64)).astype(np.float32)
    s = orc.roundtrip_stats(x, x.copy())
    assert s[0] == 0.0 and s[2] == 0.0 and s[3] == 0.0
    assert abs(s[1] - float(np.sum(x.astype(np.float64) ** 2))) <= 1e-12 * s[1]
    c = 0.125
    s = orc.roundtrip_stats(x, x.astype(np.float64) + c)
    assert abs(s[0] - x.size * c * c) <= 1e-9 and abs(s[2] - x.size * c) <= 1e-9 and s[3] == c
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # bf16 inputs by truncation
    s = orc.roundtrip_stats(bits, orc.bf16_bits_to_f64(bits))
    assert s[0] == 0.0 and s[3] == 0.0


def test_roundtrip_stats_of_sr_are_unbiased(orc):
    """The page's claim for stochastic rounding: over many seeds, the mean
    decoded error of an NVFP4 round trip goes to zero (within 5 standard
    errors plus the rule's bias bound), while round-to-nearest keeps one
    fixed error.  The tensor is a single row of one repeated block."""
    base = np.array([0.3, -1.7, 2.2, 5.1, -0.45, 0.9, 3.3, -2.6, 1.1, -0.2, 4.4, 0.05, -3.9, 2.7, -1.05, 0.6],
                     np.float32)
    x = np.tile(base, (1, 64))
    means = []
    for seed in range(200):
        c, sc, S = orc.quantize(x, orc.NVFP4, orc.SR, seed=seed, amax=6.0 * 448.0 * 0.01)
        y = orc.dequantize(orc.NVFP4, c, sc, S, 1, x.shape[1])
        means.append(orc.roundtrip_stats(x, y)[2] / x.size)
    m, se = float(np.mean(means)), float(np.std(means)) / np.sqrt(len(means))
    assert abs(m) <= 5 * se + 2.0**-16 * 2.0
    c, sc, S = orc.quantize(x, orc.NVFP4, amax=6.0 * 448.0 * 0.01)
    y = orc.dequantize(orc.NVFP4, c, sc, S, 1, x.shape[1])
    assert abs(orc.roundtrip_stats(x, y)[2] / x.size) > 10 * se
