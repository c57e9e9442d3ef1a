"""GPU parity of the matrix-instruction tile layout: tiled quantizer output
equals the oracle's row-major codes and scales after the host permutation,
tiled dequantization equals row-layout dequantization, and the tiled GEMM
(register-direct kernel) meets the same bounds as the row-layout GEMM."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import check_gemm, dev, host, to_gpu_bf16
    from tests.tiles import tile_codes, tile_scales, untile_codes, untile_scales


def _rowbytes(fmt, cols):
    return cols if fmt == 1 else cols // 2


def _quant_tiled(x_bits, fmt, rnd=0, seed=0, counter=0, rht=False, mask=0):
    R, C = x_bits.shape
    out = mx.empty(fmt, R, C, device=dev(), layout=mx.MX_LAYOUT_TILED)
    mx.mx_quantize(to_gpu_bf16(x_bits), out, rnd, seed, counter, mx.MX_FLAG_RHT16 if rht else 0, mask)
    torch.cuda.synchronize()
    c, s, _ = host(out)
    return untile_codes(c, R, _rowbytes(fmt, C)), untile_scales(s, R, C // 32)


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("rnd,rht", [(0, False), (1, False), (0, True), (1, True)])
@pytest.mark.parametrize("shape", [(32, 1024), (96, 2048), (64, 3072)])
def test_tiled_quantize_bit_exact(fmt, rnd, rht, shape):
    R, C = shape
    x = W.normal_bf16(R, C, 1.0, 3, 200, outlier_entries=0.002, outlier_mult=60)
    mask = mx.mx_rht_signs(4) if rht else 0
    c, s = _quant_tiled(x, fmt, rnd, 5, 77, rht, mask)
    wc, ws, _ = oracle.quantize(x, fmt, rnd, 5, 77, rht=rht, sign_mask=mask)
    assert np.array_equal(s, ws), "scales"
    assert np.array_equal(c, wc), "codes"


@pytest.mark.parametrize("fmt", [1, 2])
def test_tiled_dequantize_matches_rows(fmt):
    R, C = 64, 2048
    x = to_gpu_bf16(W.normal_bf16(R, C, 1.0, 4, 201))
    qt = mx.empty(fmt, R, C, device=dev(), layout=mx.MX_LAYOUT_TILED)
    qr = mx.empty(fmt, R, C, device=dev())
    mx.mx_quantize(x, qt)
    mx.mx_quantize(x, qr)
    yt = torch.empty(R, C, dtype=torch.float32, device=dev())
    yr = torch.empty(R, C, dtype=torch.float32, device=dev())
    mx.mx_dequantize(qt, yt)
    mx.mx_dequantize(qr, yr)
    torch.cuda.synchronize()
    assert torch.equal(yt.view(torch.int32), yr.view(torch.int32))


def _upload_tiled(fmt, codes, scales):
    R = codes.shape[0]
    C = codes.shape[1] * (1 if fmt == 1 else 2)
    return mx.MXTensor(fmt, R, C, torch.from_numpy(tile_codes(codes)).to(dev()),
                       torch.from_numpy(tile_scales(scales)).to(dev()), None, mx.MX_LAYOUT_TILED)


TILED_SHAPES = [(256, 256, 1024), (320, 288, 2048), (96, 544, 1024), (512, 256, 3072)]


@pytest.mark.parametrize("shape", TILED_SHAPES)
@pytest.mark.parametrize("cdt", ["f32", "bf16"])
@pytest.mark.parametrize("fmt,flags", [(2, 0), (1, 1)])
def test_tiled_gemm_within_tolerance(shape, cdt, fmt, flags):
    """MXFP4: exact products, 1e-5 bound.  MXFP8 tiled runs the native FP8
    instruction (flags=1), bound 100x (see the native-path test)."""
    M, N, K = shape
    a = W.normal_bf16(M, K, 1.0, M + K, 210, outlier_entries=0.002, outlier_mult=50)
    b = W.normal_bf16(N, K, 0.5, N + K, 211)
    qa, qb = oracle.quantize(a, fmt), oracle.quantize(b, fmt)
    A, B = _upload_tiled(fmt, qa[0], qa[1]), _upload_tiled(fmt, qb[0], qb[1])
    dt = torch.float32 if cdt == "f32" else torch.bfloat16
    C = torch.full((M, N + 5), float("nan"), dtype=dt, device=dev())[:, :N]
    mx.mx_gemm_ex(A, B, C, flags)
    torch.cuda.synchronize()
    Chat, tol = oracle.gemm(oracle.dequantize_f64(fmt, qa[0], qa[1], M, K),
                            oracle.dequantize_f64(fmt, qb[0], qb[1], N, K))
    check_gemm(C.float().cpu().numpy(), Chat, tol * (100.0 if flags else 1.0), cdt == "bf16",
               f"tiled fmt {fmt} {shape} {cdt}")


def test_tiled_quantize_then_gemm_4096_sampled():
    """The benchmark's path at full size: cfg2 operands quantized to MXFP4
    in the tile layout on the GPU, then the tiled GEMM, BF16 out; codes and
    scales bit-exact, GEMM sampled against the FP64 oracle."""
    A_bits, B_bits = W.cfg2(0, 4096)
    M = N = K = 4096
    qa = mx.empty(2, M, K, device=dev(), layout=mx.MX_LAYOUT_TILED)
    qb = mx.empty(2, N, K, device=dev(), layout=mx.MX_LAYOUT_TILED)
    mx.mx_quantize(to_gpu_bf16(A_bits), qa)
    mx.mx_quantize(to_gpu_bf16(B_bits), qb)
    C = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    mx.mx_gemm(qa, qb, C)
    torch.cuda.synchronize()
    oa, ob = oracle.quantize(A_bits, 2), oracle.quantize(B_bits, 2)
    ca, sa, _ = host(qa)
    assert np.array_equal(untile_codes(ca, M, K // 2), oa[0]) and np.array_equal(untile_scales(sa, M, K // 32), oa[1])
    g = np.random.default_rng(11)
    ri, cj = g.integers(0, M, 4096), g.integers(0, N, 4096)
    ri[:4] = [0, M - 1, 0, M - 1]
    cj[:4] = [0, 0, N - 1, N - 1]
    Chat, tol = oracle.gemm_sampled(oracle.dequantize_f64(2, oa[0], oa[1], M, K),
                                    oracle.dequantize_f64(2, ob[0], ob[1], N, K), ri, cj)
    check_gemm(C.float().cpu().numpy()[ri, cj], Chat, tol, True, "tiled 4096^3")
