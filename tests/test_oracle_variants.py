"""Pins for the oracle's quantizer variants: the ceil (no-saturation) E8M0 rule,
the Four Over Six NVFP4 block-scale choice and 2-D (16 x 16) NVFP4 blocks.

Each variant is tied to something other than its own code: hand-worked
blocks (tests/golden/), boundary cases that separate < from <=, and exact
relations to the plain quantizers, which have their own pins."""
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _fp4_codes(codes, cols):
    """uint8 [rows, cols/2] -> int [rows, cols] (element 2j in the low nibble)."""
    lo = codes & 0xF
    hi = codes >> 4
    out = np.empty((codes.shape[0], cols), np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


# --- ceil E8M0 rule -----------------------------------------------------------
def test_ceil_rule_worked_example(orc):
    """A block maximum of 3.7 in MXFP4: the floor rule saturates it to 3, the
    ceil rule keeps the whole block in range and decodes it to 4."""
    want = {r[0]: (int(r[1]), int(r[2]), float(r[3])) for r in _read_rows("mxfp4_scale_choice.txt")}
    x = np.zeros((1, 32), np.float32)
    x[0, 3] = 3.7
    x[0, 9] = 1.0
    for rule, variant in (("floor", 0), ("ceil", orc.V_CEIL)):
        codes, scales, _ = orc.quantize(x, orc.MXFP4, variant=variant)
        sc, mc, dmax = want[rule]
        assert int(scales[0, 0]) == sc
        assert _fp4_codes(codes, 32)[0, 3] == mc
        y = orc.dequantize(orc.MXFP4, codes, scales, None, 1, 32)
        assert float(y[0, 3]) == dmax


@pytest.mark.parametrize("fmt,gmax,emax", [(1, 448.0, 8), (2, 6.0, 2)])
def test_ceil_rule_boundaries(orc, fmt, gmax, emax):
    """A block maximum of exactly g_max * 2^k keeps the floor scale (k);
    the next FP32 value above it needs k + 1.  Maxima whose significand is at
    most g_max's share the floor code."""
    for k in (-120, -30, -1, 0, 3, 40, 100):
        for amax, want_e in ((gmax * 2.0 ** k, k),
                             (float(np.nextafter(np.float32(gmax * 2.0 ** k), np.float32(np.inf))), k + 1),
                             (2.0 ** (k + emax), k)):
            x = np.zeros((1, 32), np.float32)
            x[0, 17] = -amax
            x[0, 2] = amax / 3
            _, s_ceil, _ = orc.quantize(x, fmt, variant=orc.V_CEIL)
            assert int(s_ceil[0, 0]) == want_e + 127, (k, amax)


@pytest.mark.parametrize("fmt", [1, 2])
def test_ceil_rule_versus_floor_rule(orc, fmt):
    """On random blocks over a wide range: the ceil code is the floor code or
    the floor code + 1, and it is + 1 exactly when the floor rule saturates
    the block maximum (its decoded maximum falls short of max|x| by more
    than rounding allows); with the ceil rule nothing saturates."""
    gmax = 448.0 if fmt == orc.MXFP8 else 6.0
    g = np.random.default_rng(11)
    x = (g.standard_normal((96, 256)) * np.exp(g.uniform(-30, 30, (96, 1)))).astype(np.float32)
    cf, sf, _ = orc.quantize(x, fmt)
    cc, scl, _ = orc.quantize(x, fmt, variant=orc.V_CEIL)
    d = scl.astype(np.int64) - sf.astype(np.int64)
    assert set(np.unique(d)) <= {0, 1}
    amax = np.abs(x.astype(np.float64)).reshape(96, 8, 32).max(axis=2)
    sat_floor = amax * 2.0 ** -(sf.astype(np.float64) - 127) > gmax
    assert np.array_equal(d == 1, sat_floor)
    assert sat_floor.any() and (~sat_floor).any()
    assert np.all(amax * 2.0 ** -(scl.astype(np.float64) - 127) <= gmax)
    # blocks with the same code are encoded identically
    same = np.repeat(d == 0, 32, axis=1)
    yf = orc.dequantize(fmt, cf, sf, None, 96, 256)
    yc = orc.dequantize(fmt, cc, scl, None, 96, 256)
    assert np.array_equal(yf[same], yc[same])


def test_ceil_rule_makes_sr_unbiased_at_the_block_max(orc):
    """Stochastic rounding keeps the mean only when nothing saturates: with the
    floor rule a block maximum of 7.4 * 2^-1 is always cut to 3; with the ceil
    rule its draws average to 3.7 (many independent rows of one block)."""
    n = 4000
    x = np.zeros((n, 32), np.float32)
    x[:, 0] = 3.7
    x[:, 1] = 1.0
    for variant, want, tol in ((0, 3.0, 1e-12), (orc.V_CEIL, 3.7, 0.03)):
        c, s, _ = orc.quantize(x, orc.MXFP4, rnd=orc.SR, seed=3, variant=variant)
        y = orc.dequantize(orc.MXFP4, c, s, None, n, 32)
        assert abs(float(y[:, 0].mean()) - want) <= tol


# --- Four Over Six ------------------------------------------------------------
def test_four_over_six_worked_blocks(orc):
    rows = {r[0]: (int(r[1], 16), [int(v) for v in r[2:]]) for r in _read_rows("nvfp4_four_over_six.txt")}
    x = np.zeros((1, 48), np.float32)
    x[0, 0:16] = 48.0
    x[0, 0] = 64.0
    x[0, 16:32] = 16.0
    x[0, 16] = 96.0
    x[0, 32] = 12.0
    x[0, 33] = 6.0
    codes, scales, S = orc.quantize(x, orc.NVFP4, amax=2688.0, variant=orc.V_FOUR6)
    assert S == 1.0
    c = _fp4_codes(codes, 48)
    for b, name in enumerate("ABC"):
        sc, cw = rows[name]
        assert int(scales[0, b]) == sc, name
        assert list(c[0, 16 * b:16 * b + 16]) == cw, name
    codes, scales, _ = orc.quantize(x, orc.NVFP4, amax=2688.0)
    sc, cw = rows["standard_A"]
    assert int(scales[0, 0]) == sc
    assert list(_fp4_codes(codes, 48)[0, :16]) == cw


# Exact error sums with Python's rational arithmetic, from the pages' E2M1
# alphabet ("08 - FP4, MXFP4, NVFP4", "Why 4-bit floats at all?") and torch's
# E4M3 decoder: independent of the oracle's big-integer sums.
_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e4m3_value(code):
    import torch
    return float(torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


def _decoded_f32(code, sb, S):
    p = np.float32((-1.0 if code & 8 else 1.0) * _E2M1[code & 7] * _e4m3_value(sb))  # exact
    return np.float32(p * np.float32(S))


def _exact_err(v, codes, sb, S):
    from fractions import Fraction as Fr
    return sum((Fr(float(v[j])) - Fr(float(_decoded_f32(int(codes[j]), sb, S)))) ** 2 for j in range(16))


def _f32_round(q):
    """Correctly rounded (nearest, ties to even) FP32 value of a rational q."""
    from fractions import Fraction as Fr
    if q == 0:
        return np.float32(0.0)
    sgn, q = (-1 if q < 0 else 1), abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fr(2) ** e > q:
        e -= 1
    while Fr(2) ** (e + 1) <= q:
        e += 1
    ulp = Fr(2) ** (max(e, -126) - 23)
    m = q / ulp
    fl = m.numerator // m.denominator
    if m - fl > Fr(1, 2) or (m - fl == Fr(1, 2) and fl % 2):
        fl += 1
    return np.float32(sgn * float(fl * ulp))


def _old_fp32_err(v, codes, sb, S):
    """The former definition: two FP32 halves of 8 accumulated with fused
    multiply-adds (one rounding each), then added in FP32."""
    from fractions import Fraction as Fr
    half = [np.float32(0.0), np.float32(0.0)]
    for j in range(16):
        d = np.float32(v[j] - _decoded_f32(int(codes[j]), sb, S))
        half[j // 8] = _f32_round(Fr(float(d)) ** 2 + Fr(float(half[j // 8])))
    return np.float32(half[0] + half[1])


def _near_tie_blocks():
    u, v = 2.0 ** -12, 4095 * 2.0 ** -22
    D = [24.0] + [21.0] * 6 + [3 + u] + [21.0] * 7 + [2 + u + 2.0 ** -22]
    E = [24.0, 21.0, 21.0, 3 + v, 0, 0, 0, 0, 21.0, 2 + v - 2.0 ** -22, 0, 0, 0, 0, 0, 0]
    return np.array([D, E], np.float32)


def test_four_over_six_near_ties(orc):
    """Blocks D and E of the golden file: the exact comparison keeps 4 for D and
    6 for E, by 2^-21; the former FP32 order decided both the other way."""
    from fractions import Fraction as Fr
    rows = {r[0]: (int(r[1], 16), [int(v) for v in r[2:]]) for r in _read_rows("nvfp4_four_over_six.txt")}
    x = _near_tie_blocks()
    codes, scales, S = orc.quantize(x, orc.NVFP4, amax=2688.0, variant=orc.V_FOUR6)
    c0, s0, _ = orc.quantize(x, orc.NVFP4, amax=2688.0)
    assert S == 1.0
    c, k0 = _fp4_codes(codes, 16), _fp4_codes(c0, 16)
    for i, name in enumerate("DE"):
        sc, cw = rows[name]
        assert int(scales[i, 0]) == sc and list(c[i]) == cw, name
    # the two candidates of each block, and their exact errors
    c4 = [6] * 7 + [1] + [6] * 7 + [1]
    assert list(k0[0]) == [7] * 7 + [2] + [7] * 7 + [1] and list(c[0]) == c4
    for i, (want, sign) in enumerate(((0x4C, 1), (0x48, -1))):
        six = (int(s0[i, 0]), k0[i])
        four = (0x4C, c4 if i == 0 else [6, 6, 6, 1, 0, 0, 0, 0, 6, 1, 0, 0, 0, 0, 0, 0])
        d = _exact_err(x[i], six[1], six[0], 1.0) - _exact_err(x[i], four[1], four[0], 1.0)
        assert d == sign * Fr(1, 2 ** 21)
        assert orc.nv_sq_error_cmp(x[i], six[1], six[0], four[1], four[0], 1.0) == sign
        old6, old4 = _old_fp32_err(x[i], six[1], six[0], 1.0), _old_fp32_err(x[i], four[1], four[0], 1.0)
        assert (old4 < old6) == (sign < 0), "the FP32 order must decide this block the other way"


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_four_over_six_exact_comparison(orc, seed):
    """The oracle's integer error sums against rational arithmetic, on random
    FP32 blocks whose values span a wide range of magnitudes (subnormal to
    2^100) and on near-tie blocks built like D and E with random perturbations."""
    g = np.random.default_rng(seed)
    n = 0
    for t in range(300):
        if t % 3 == 0:
            v = (g.standard_normal(16) * np.exp2(g.integers(-140, 100, 16))).astype(np.float32)
        elif t % 3 == 1:
            v = (g.standard_normal(16) * 2.0 ** float(g.integers(-130, 120))).astype(np.float32)
        else:
            e, f = g.integers(1, 1 << 12, 2) * 2.0 ** -22
            v = np.array([24.0] + [21.0] * 6 + [3 + e] + [21.0] * 7 + [2 + f], np.float32)
            v *= np.float32(2.0 ** float(g.integers(-20, 20)))
        S = np.float32(np.abs(v).max() / 2688.0 * float(g.choice([1.0, 1.5, 4.0])))
        if S == 0 or not np.isfinite(S):
            continue
        ca = g.integers(0, 16, 16).astype(np.uint8)
        cb = ca.copy()
        cb[g.integers(0, 16, 3)] = g.integers(0, 16, 3)
        sa, sbb = int(g.integers(0, 0x7F)), int(g.integers(0, 0x7F))
        want = _exact_err(v, ca, sa, S) - _exact_err(v, cb, sbb, S)
        got = orc.nv_sq_error_cmp(v, ca, sa, cb, sbb, float(S))
        assert got == (want > 0) - (want < 0), (t, v, ca, sa, cb, sbb, S)
        assert orc.nv_sq_error_cmp(v, ca, sa, ca, sa, float(S)) == 0
        n += 1
    assert n > 250


def _block_sq_err(x, y):
    d = (x.astype(np.float64) - y.astype(np.float64)) ** 2
    return d.reshape(x.shape[0], -1, 16).sum(axis=2)


@pytest.mark.parametrize("seed", [0, 1])
def test_four_over_six_versus_standard(orc, seed):
    """Every block either keeps the plain NVFP4 encoding bit for bit, or has a
    block scale equal to the E4M3 rounding of max|x| / (4 S) (torch's E4M3
    cast, an independent routine), its largest element code 4, and a
    smaller error than the plain encoding.  Overall error drops."""
    import torch
    g = np.random.default_rng(seed)
    x = g.standard_normal((64, 512)).astype(np.float32)
    x[g.random(x.shape) < 0.01] *= 20
    c0, s0, S0 = orc.quantize(x, orc.NVFP4)
    c1, s1, S1 = orc.quantize(x, orc.NVFP4, variant=orc.V_FOUR6)
    assert S0 == S1
    y0 = orc.dequantize(orc.NVFP4, c0, s0, S0, 64, 512)
    y1 = orc.dequantize(orc.NVFP4, c1, s1, S1, 64, 512)
    e0, e1 = _block_sq_err(x, y0), _block_sq_err(x, y1)
    k0, k1 = _fp4_codes(c0, 512).reshape(64, 32, 16), _fp4_codes(c1, 512).reshape(64, 32, 16)
    kept = (s0 == s1) & np.all(k0 == k1, axis=2)
    changed = ~kept
    assert 0.1 < changed.mean() < 0.9
    ab = np.abs(x).reshape(64, 32, 16).max(axis=2)
    d4 = np.float32(4.0) * np.float32(S1)
    q4 = (ab / d4).astype(np.float32)
    sb4 = torch.from_numpy(q4).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s1[changed], sb4[changed])
    assert np.all((k1 & 7).max(axis=2)[changed] == 6)
    assert np.all(e1[changed] <= e0[changed] * (1 + 1e-6))
    assert e1.sum() < e0.sum()


def test_four_over_six_zero_and_degenerate(orc):
    """All-zero tensor and all-zero blocks: the plain encoding (ties keep 6).
    SR and the 2-D variant are rejected."""
    x = np.zeros((2, 32), np.float32)
    c, s, S = orc.quantize(x, orc.NVFP4, variant=orc.V_FOUR6)
    assert S == 1.0 and not c.any() and not s.any()
    x[0, :16] = np.linspace(-3, 3, 16)
    c1, s1, _ = orc.quantize(x, orc.NVFP4, variant=orc.V_FOUR6)
    c0, s0, _ = orc.quantize(x, orc.NVFP4)
    assert np.array_equal(c1[:, 8:], c0[:, 8:]) and np.array_equal(s1[:, 1], s0[:, 1])
    with pytest.raises(ValueError):
        orc.quantize(x, orc.NVFP4, rnd=orc.SR, variant=orc.V_FOUR6)
    with pytest.raises(ValueError):
        orc.quantize(x, orc.NVFP4, variant=orc.V_FOUR6 | orc.V_2D)


# --- 2-D blocks ---------------------------------------------------------------
def _weights(g, rows, cols):
    w = (g.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w *= np.exp(g.uniform(-2, 2, (rows, 1))).astype(np.float32)
    return w


def test_2d_blocks_commute_with_transpose(orc):
    """The quantized values of W^T are the transpose of those of W."""
    g = np.random.default_rng(4)
    w = _weights(g, 96, 160)
    c, s, S = orc.quantize(w, orc.NVFP4, variant=orc.V_2D)
    ct, st, St = orc.quantize(np.ascontiguousarray(w.T), orc.NVFP4, variant=orc.V_2D)
    assert S == St
    y = orc.dequantize(orc.NVFP4, c, s, S, 96, 160)
    yt = orc.dequantize(orc.NVFP4, ct, st, St, 160, 96)
    assert np.array_equal(y.T, yt)
    # the plain 1-D encoding does not have this property on such data
    c1, s1, S1 = orc.quantize(w, orc.NVFP4)
    c1t, s1t, _ = orc.quantize(np.ascontiguousarray(w.T), orc.NVFP4)
    assert not np.array_equal(orc.dequantize(orc.NVFP4, c1, s1, S1, 96, 160).T,
                              orc.dequantize(orc.NVFP4, c1t, s1t, S1, 160, 96))


@pytest.mark.parametrize("rows,rnd", [(64, 0), (53, 0), (37, 1)])
def test_2d_scale_is_band_max_of_1d_scales(orc, rows, rnd):
    """E4M3 rounding is monotone, so a 16 x 16 tile's scale code is the largest
    of the 1-D codes of its rows (the last band may be short); rows whose 1-D
    code already equals it are encoded identically, random draws included."""
    g = np.random.default_rng(rows)
    w = _weights(g, rows, 128)
    c2, s2, S2 = orc.quantize(w, orc.NVFP4, rnd=rnd, seed=9, variant=orc.V_2D)
    c1, s1, S1 = orc.quantize(w, orc.NVFP4, rnd=rnd, seed=9)
    assert S1 == S2
    for r0 in range(0, rows, 16):
        band = s1[r0:r0 + 16].astype(np.int64)
        assert np.array_equal(s2[r0:r0 + 16], np.broadcast_to(band.max(axis=0), band.shape))
    k1, k2 = _fp4_codes(c1, 128).reshape(rows, 8, 16), _fp4_codes(c2, 128).reshape(rows, 8, 16)
    same = s1 == s2
    assert np.array_equal(k1[same], k2[same])
    assert (~same).any()


def test_2d_equal_rows_reduce_to_1d(orc):
    g = np.random.default_rng(8)
    base = _weights(g, 4, 64)
    w = np.repeat(base, 16, axis=0)
    a = orc.quantize(w, orc.NVFP4, variant=orc.V_2D)
    b = orc.quantize(w, orc.NVFP4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


# --- vectorised element encoder (used by the fused quantize-GEMM checks) -------
@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("rnd", [0, 1])
def test_encode_elems_equals_the_scalar_encoders(orc, fmt, rnd):
    g = np.random.default_rng(fmt + 2 * rnd)
    y = g.standard_normal(300) * (100.0 if fmt == 1 else 3.0)
    y[:4] = [0.0, -0.0, 1e9, -1e9]
    n = g.integers(0, 1 << 40, 300).astype(np.uint64)
    got = orc.encode_elems(fmt, y, rnd, n, seed=7, counter=11)
    if rnd == 0:
        enc = orc.e4m3_encode_rne if fmt == 1 else orc.e2m1_encode_rne
        want = [enc(float(v)) for v in y]
    else:
        enc = orc.e4m3_encode_sr if fmt == 1 else orc.e2m1_encode_sr
        want = [enc(float(v), orc.rand16(7, 11, int(k))) for v, k in zip(y, n)]
    assert list(got) == want
