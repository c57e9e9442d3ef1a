"""Pins for the FP64 GEMM oracle: exact rational arithmetic on tiny shapes,
the identity closed form and power-of-two scale invariance."""
from fractions import Fraction

import numpy as np

import workloads as W


def test_gemm_exact_rational_tiny(orc):
    g = np.random.default_rng(20)
    for fmt in (orc.MXFP8, orc.MXFP4, orc.NVFP4):
        M, N, K = 5, 7, 64
        A = W.normal_bf16(M, K, seed=5, tensor_id=fmt)
        B = W.normal_bf16(N, K, seed=6, tensor_id=fmt)
        qa = orc.quantize(A, fmt)
        qb = orc.quantize(B, fmt)
        Ad = orc.dequantize_f64(fmt, qa[0], qa[1], M, K)
        Bd = orc.dequantize_f64(fmt, qb[0], qb[1], N, K)
        post = 1.0
        if fmt == orc.NVFP4:
            post = float(np.float32(qa[2]) * np.float32(qb[2]))
        C, T = orc.gemm(Ad, Bd, post)
        for i in range(M):
            for j in range(N):
                s = sum(Fraction(Ad[i, k]) * Fraction(Bd[j, k]) for k in range(K))
                sa = sum(abs(Fraction(Ad[i, k]) * Fraction(Bd[j, k])) for k in range(K))
                exact = s * Fraction(post)
                assert abs(Fraction(C[i, j]) - exact) <= abs(exact) * Fraction(1, 2**50) + Fraction(1, 2**1000)
                assert abs(Fraction(T[i, j]) - Fraction(1, 100000) * sa * abs(Fraction(post))) <= sa * Fraction(1, 2**45)


def test_gemm_identity_closed_form(orc):
    """A coded as the identity (code 1.0 on the diagonal, scale 2^0) gives
    C = B-hat transposed exactly."""
    K = 64
    eye = np.eye(K, dtype=np.float32)
    qa = orc.quantize(eye, orc.MXFP8)
    # block holding the 1.0: max 1 -> X = 2^(0-8) (1.0 stored as 256); the
    # all-zero block of each row gets the smallest scale, code 0
    want = np.zeros((K, K // 32), np.uint8)
    want[np.arange(K), np.arange(K) // 32] = 127 - 8
    assert np.array_equal(qa[1], want)
    B = W.normal_bf16(9, K, seed=7, tensor_id=1)
    qb = orc.quantize(B, orc.MXFP4)
    Ad = orc.dequantize_f64(orc.MXFP8, qa[0], qa[1], K, K)
    assert np.array_equal(Ad, np.eye(K))
    Bd = orc.dequantize_f64(orc.MXFP4, qb[0], qb[1], 9, K)
    C, _ = orc.gemm(Ad, Bd)
    assert np.array_equal(C, Bd.T)


def test_gemm_power_of_two_scale_invariance(orc):
    M, N, K = 8, 8, 96
    A = W.normal_bf16(M, K, seed=8, tensor_id=1)
    B = W.normal_bf16(N, K, seed=8, tensor_id=2)
    qa = orc.quantize(A, orc.MXFP4)
    qb = orc.quantize(B, orc.MXFP4)
    Ad = orc.dequantize_f64(orc.MXFP4, qa[0], qa[1], M, K)
    Bd = orc.dequantize_f64(orc.MXFP4, qb[0], qb[1], N, K)
    C, _ = orc.gemm(Ad, Bd)
    sa = qa[1].astype(np.int32) + 3
    sb = qb[1].astype(np.int32) - 5
    Ad2 = orc.dequantize_f64(orc.MXFP4, qa[0], sa.astype(np.uint8), M, K)
    Bd2 = orc.dequantize_f64(orc.MXFP4, qb[0], sb.astype(np.uint8), N, K)
    C2, _ = orc.gemm(Ad2, Bd2)
    assert np.array_equal(C2, C * 2.0 ** -2)


def test_gemm_sampled_matches_full(orc):
    g = np.random.default_rng(21)
    A = g.standard_normal((33, 64))
    B = g.standard_normal((17, 64))
    C, T = orc.gemm(A, B)
    ri = g.integers(0, 33, 50)
    cj = g.integers(0, 17, 50)
    Cs, Ts = orc.gemm_sampled(A, B, ri, cj)
    assert np.array_equal(Cs, C[ri, cj]) and np.array_equal(Ts, T[ri, cj])


def test_bf16_interval_rounding(orc):
    # exact bf16 values map to themselves; midpoints round to even
    v = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -3.0, 2.0**-130, 0.0])
    r = orc._round_bf16_f64(v)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 * 2**-7 and r[3] == -3.0
    assert r[5] == 0.0
    # against torch's float32 -> bf16 RNE for values exactly representable in FP32
    import torch
    x = np.random.default_rng(22).standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc._round_bf16_f64(x.astype(np.float64)), ref)


def test_f32_interval(orc):
    """The FP32 acceptance interval is the plain bound where C +- tol are FP32
    values, and the FP32 rounding of C when the bound is narrower than FP32's
    spacing (subnormal results, results below 2^-149)."""
    C = np.array([1.0, -3.5, 2.0**-140, 2.0**-140 + 2.0**-170, 2.0**-200, -(2.0**-151) * 3])
    tol = np.array([2.0**-10, 2.0**-8, 2.0**-157, 2.0**-187, 2.0**-217, 2.0**-170])
    lo, hi = orc.f32_interval(C, tol)
    assert lo[0] == 1.0 - 2.0**-10 and hi[0] == 1.0 + 2.0**-10
    assert lo[1] == -3.5 - 2.0**-8 and hi[1] == -3.5 + 2.0**-8
    assert lo[2] == hi[2] == 2.0**-140
    assert lo[3] == hi[3] == 2.0**-140
    assert lo[4] == hi[4] == 0.0
    assert lo[5] == hi[5] == -(2.0**-149)  # three quarters of a spacing rounds to one spacing
