"""GPU checks of the GEMM whose output is written quantized (mx_gemm_quantize).

The FP32 product C = A * B^T is fixed only to within the GEMM bound, so its
quantization is not unique near rounding and scale boundaries.  The oracle is
the composition of its pinned pieces -- exact FP64 product and tolerance, then
the MX scale rule and element encoders -- and the check is that the kernel's
output is the quantization of SOME matrix inside the bound:
  * each block's scale code lies between the codes of the smallest and the
    largest block maximum the bound allows;
  * given that scale, each element's code lies between the encodings of
    (C - tol) / X and (C + tol) / X -- both encoders are monotone, SR with the
    element's own random value (its row-major index in C).
Where the interval holds one code (most elements) that code is unique and the
check is exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import dev
    from tests.tiles import tile_codes, tile_scales, untile_codes, untile_scales


def _elems(fmt, codes, cols):
    if fmt in (oracle.MXFP8, oracle.MXFP8_E5M2):
        return codes.astype(np.int64)
    out = np.empty((codes.shape[0], cols), np.int64)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def _dec(fmt, codes):
    if fmt == oracle.MXFP8_E5M2:
        lut = np.array([oracle.elem_decode(fmt, c) for c in range(256)], np.float64)
        return lut[codes]
    f = oracle.e4m3_decode if fmt == oracle.MXFP8 else oracle.e2m1_decode
    lut = np.array([f(c) for c in range(256 if fmt == oracle.MXFP8 else 16)], np.float64)
    return lut[codes]


def _scale_codes(fmt, amax_f32, ceil):
    """Oracle scale codes of blocks with the given maxima (one block per row)."""
    x = np.zeros((amax_f32.size, 32), np.float32)
    x[:, 0] = amax_f32
    _, s, _ = oracle.quantize(x, fmt, variant=oracle.V_CEIL if ceil else 0)
    return s[:, 0].astype(np.int64)


def check_quantized_product(C, tol, ofmt, codes, scales, rnd, seed, counter, ceil, rows_idx=None):
    """C, tol: FP64 [R, N] oracle product rows (rows_idx: their row numbers in
    the full product, default 0..R-1); codes/scales: the kernel's output rows
    in the row layout."""
    R, N = C.shape
    rows_idx = np.arange(R) if rows_idx is None else np.asarray(rows_idx)
    nb = N // 32
    sc = scales.astype(np.int64)
    Cb, Tb = C.reshape(R, nb, 32), tol.reshape(R, nb, 32)
    amax_lo = np.maximum(np.abs(Cb) - Tb, 0.0).max(axis=2)
    amax_hi = (np.abs(Cb) + Tb).max(axis=2)
    lo32 = np.nextafter(amax_lo.astype(np.float32), np.float32(0))
    lo32 = np.where(amax_lo == 0, np.float32(0), lo32)
    hi32 = np.nextafter(amax_hi.astype(np.float32), np.float32(np.inf))
    c_lo = _scale_codes(ofmt, lo32.ravel(), ceil).reshape(R, nb)
    c_hi = _scale_codes(ofmt, hi32.ravel(), ceil).reshape(R, nb)
    bad = (sc < c_lo) | (sc > c_hi)
    assert not bad.any(), f"{int(bad.sum())} block scales outside their interval, first at {np.argwhere(bad)[:3]}"
    X = np.repeat(2.0 ** (sc - 127).astype(np.float64), 32, axis=1)
    n = (rows_idx[:, None].astype(np.uint64) * np.uint64(N) + np.arange(N, dtype=np.uint64)[None, :])
    e_lo = oracle.encode_elems(ofmt, (C - tol) / X, rnd, n, seed, counter).reshape(R, N)
    e_hi = oracle.encode_elems(ofmt, (C + tol) / X, rnd, n, seed, counter).reshape(R, N)
    got = _dec(ofmt, _elems(ofmt, codes, N))
    v_lo, v_hi = _dec(ofmt, e_lo.astype(np.int64)), _dec(ofmt, e_hi.astype(np.int64))
    bad = (got < v_lo) | (got > v_hi)
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} elements outside their interval, first at "
                           f"{np.argwhere(bad)[:3]}")
    return float(np.mean(v_lo == v_hi))


def _operands(M, N, K, fmt, seed):
    a = W.normal_bf16(M, K, 1.0, seed, 70, outlier_entries=0.002, outlier_mult=40.0)
    b = W.normal_bf16(N, K, 0.05, seed, 71)
    qa = oracle.quantize(a, fmt)
    qb = oracle.quantize(b, fmt)
    return qa, qb


def _upload_tiled(fmt, q, rows, cols):
    c, s, _ = q
    return mx.MXTensor(fmt, rows, cols, torch.from_numpy(tile_codes(c)).to(dev()),
                       torch.from_numpy(tile_scales(s)).to(dev()), None, mx.MX_LAYOUT_TILED)


def _run(M, N, K, fmt, ofmt, rnd, otiled, ceil, seed):
    qa, qb = _operands(M, N, K, fmt, seed)
    A = _upload_tiled(fmt, qa, M, K)
    B = _upload_tiled(fmt, qb, N, K)
    out = mx.empty(ofmt, M, N, device=dev(), layout=mx.MX_LAYOUT_TILED if otiled else mx.MX_LAYOUT_ROWS)
    flags = (mx.MX_FLAG_SCALE_CEIL if ceil else 0) | (mx.MX_GEMM_FP8_NATIVE if fmt == oracle.MXFP8 else 0)
    mx.mx_gemm_quantize(A, B, out, rnd, seed, 5 * seed + 1, flags)
    torch.cuda.synchronize()
    codes, scales = out.codes.cpu().numpy(), out.scales.cpu().numpy()
    rb = N if ofmt in (oracle.MXFP8, oracle.MXFP8_E5M2) else N // 2
    if otiled:
        codes, scales = untile_codes(codes, M, rb), untile_scales(scales, M, N // 32)
    return qa, qb, codes.reshape(M, rb), scales.reshape(M, N // 32)


@pytest.mark.parametrize("ofmt", [1, 2, 5])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("otiled", [False, True])
def test_quantized_product_mxfp4(ofmt, rnd, otiled):
    M, N, K = 256, 1024, 2048
    seed = 3 + ofmt + 2 * rnd
    qa, qb, codes, scales = _run(M, N, K, 2, ofmt, rnd, otiled, False, seed)
    Ad = oracle.dequantize_f64(2, qa[0], qa[1], M, K)
    Bd = oracle.dequantize_f64(2, qb[0], qb[1], N, K)
    C, tol = oracle.gemm(Ad, Bd)
    unique = check_quantized_product(C, tol, ofmt, codes, scales, rnd, seed, 5 * seed + 1, False)
    assert unique > 0.95


@pytest.mark.parametrize("shape", [(96, 64, 1024), (288, 1056, 1024), (544, 2048, 3072)])
@pytest.mark.parametrize("ceil", [False, True])
def test_quantized_product_ragged_and_ceil(shape, ceil):
    """Tiles past M and N, several workgroup tiles, the ceil rule."""
    M, N, K = shape
    otiled = M % 32 == 0 and N % 1024 == 0
    qa, qb, codes, scales = _run(M, N, K, 2, 2, 0, otiled, ceil, 9)
    C, tol = oracle.gemm(oracle.dequantize_f64(2, qa[0], qa[1], M, K),
                         oracle.dequantize_f64(2, qb[0], qb[1], N, K))
    check_quantized_product(C, tol, 2, codes, scales, 0, 9, 46, ceil)


def test_quantized_product_native_fp8_operands():
    """MXFP8 operands on the FP8 instruction: the bound is that flag's
    1e-3 * sum|a*b|."""
    M, N, K = 256, 1024, 1024
    qa, qb, codes, scales = _run(M, N, K, 1, 2, 1, False, False, 4)
    C, tol = oracle.gemm(oracle.dequantize_f64(1, qa[0], qa[1], M, K),
                         oracle.dequantize_f64(1, qb[0], qb[1], N, K))
    check_quantized_product(C, tol * 100, 2, codes, scales, 1, 4, 21, False)


def test_quantized_product_matches_gemm_then_quantize():
    """Against the library's own two-step path on the GPU (FP32 product, then
    the quantizer): the fused codes may differ only where the FP32 product
    itself can differ, i.e. they agree almost everywhere."""
    M, N, K = 512, 2048, 2048
    qa, qb = _operands(M, N, K, 2, 12)
    A, B = _upload_tiled(2, qa, M, K), _upload_tiled(2, qb, N, K)
    fused = mx.empty(2, M, N, device=dev())
    mx.mx_gemm_quantize(A, B, fused, mx.MX_SR, 12, 0)
    C32 = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm(A, B, C32)
    two = mx.empty(2, M, N, device=dev())
    mx.mx_quantize(C32, two, mx.MX_SR, 12, 0)
    torch.cuda.synchronize()
    same_s = (fused.scales == two.scales).float().mean().item()
    same_c = (fused.codes == two.codes).float().mean().item()
    assert same_s == 1.0 and same_c == 1.0, (same_s, same_c)


def test_quantized_product_full_size_sampled_rows():
    """The 4096^3 MXFP4 product written as MXFP4 (tile layout), checked on 48
    sampled rows against the oracle's exact product."""
    M = N = K = 4096
    qa, qb, codes, scales = _run(M, N, K, 2, 2, 0, True, False, 1)
    Ad = oracle.dequantize_f64(2, qa[0], qa[1], M, K)
    Bd = oracle.dequantize_f64(2, qb[0], qb[1], N, K)
    rows = np.sort(np.random.default_rng(1).choice(M, 48, replace=False))
    ri = np.repeat(rows, N).astype(np.int64)
    cj = np.tile(np.arange(N), rows.size).astype(np.int64)
    C, tol = oracle.gemm_sampled(Ad, Bd, ri, cj)
    check_quantized_product(C.reshape(rows.size, N), tol.reshape(rows.size, N), 2, codes[rows],
                            scales[rows], 0, 1, 6, False, rows_idx=rows)


def test_quantized_product_argument_checks():
    a = mx.empty(2, 64, 1024, device=dev())  # row layout: not accepted
    out = mx.empty(2, 64, 64, device=dev())
    with pytest.raises(mx.MXError):
        mx.mx_gemm_quantize(a, a, out)
    at = mx.empty(2, 64, 1024, device=dev(), layout=mx.MX_LAYOUT_TILED)
    nv = mx.empty(3, 64, 64, device=dev())
    with pytest.raises(mx.MXError):
        mx.mx_gemm_quantize(at, at, nv)
    with pytest.raises(mx.MXError):
        mx.mx_gemm_quantize(at, at, out, flags=mx.MX_GEMM_FP8_NATIVE)
