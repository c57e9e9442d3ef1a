"""GPU parity of the other MX element types (INT8 / S2F6, FP8 E5M2, FP6 E3M2
and E2M3) against the CPU oracle: bit-exact codes and scales from the
quantizer (both input dtypes, RNE and SR, the Hadamard transform, the ceil
rule, strided inputs, ragged tails), bit-exact decoding, and the S2F6 combine
codec (Hadamard transform + block-scaled INT8, then decode + inverse
transform) at the mixture-of-experts combine size."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import dev, host, to_gpu_bf16, to_gpu_f32, upload

FMTS = [4, 5, 6, 7]
SHAPES = [(1, 32), (7, 96), (33, 256), (130, 544)]


def _inputs(rows, cols, dt, seed, pad=0, spread=False):
    bits = W.normal_bf16(rows, cols, 1.5, seed, 80, outlier_entries=0.01, outlier_mult=60.0)
    x = W.bf16_bits_to_f32(bits).astype(np.float64)
    if spread:
        x *= np.exp2(np.round(W.rng(seed, 81).uniform(-30, 30, (rows, 1))))
    if dt == "bf16":
        b = W.f64_to_bf16_bits(x)
        return b, to_gpu_bf16(b, pad)
    f = (x.astype(np.float32) * np.float32(1.0 + 2.0**-12)).astype(np.float32)
    return f, to_gpu_f32(f, pad)


def _quant(x, fmt, rnd=0, seed=0, counter=0, flags=0, mask=0):
    rows, cols = x.shape
    out = mx.empty(fmt, rows, cols, device=dev())
    mx.mx_quantize(x, out, rnd, seed, counter, flags, mask)
    torch.cuda.synchronize()
    return out


def _same(got, want, what):
    assert np.array_equal(got, want), f"{what} differ at {np.argwhere(got != want)[:5]}"


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_quantize_bit_exact(shape, fmt, rnd, rht, dt):
    rows, cols = shape
    seed = rows * 11 + cols + 3 * fmt + rnd
    x_np, x = _inputs(rows, cols, dt, seed, pad=16 if rows % 2 else 0, spread=not rht)
    mask = oracle.rht_signs(seed)
    out = _quant(x, fmt, rnd, seed, 7 * seed, mx.MX_FLAG_RHT16 if rht else 0, mask)
    c, s, _ = host(out)
    wc, ws, _ = oracle.quantize(x_np, fmt, rnd, seed, 7 * seed, rht=rht, sign_mask=mask)
    _same(s, ws, "scales")
    _same(c, wc, "codes")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rnd", [0, 1])
def test_quantize_ceil_rule_bit_exact(fmt, rnd):
    x_np, x = _inputs(64, 512, "f32", 5 + fmt, spread=True)
    out = _quant(x, fmt, rnd, 3, 1, mx.MX_FLAG_SCALE_CEIL)
    c, s, _ = host(out)
    wc, ws, _ = oracle.quantize(x_np, fmt, rnd, 3, 1, variant=oracle.V_CEIL)
    _same(s, ws, "scales")
    _same(c, wc, "codes")


@pytest.mark.parametrize("ceil", [False, True])
def test_int8_block_maxima_near_the_fp32_limit(ceil):
    """INT8's emax is 0, so maxima of 2^127 and above need scale code 254 (and
    the ceil rule clamps there); zero and NaN blocks as for the other formats."""
    x = np.zeros((4, 64), np.float32)
    x[0, :32] = np.linspace(-3e38, 3.3e38, 32, dtype=np.float32)
    x[0, 32:] = np.float32(1.7e38)
    x[1, :32] = np.float32(2.0**127)
    x[1, 5] = np.float32(-(2.0**127) * 1.5)
    x[2, 32:] = np.float32(1e-38)
    x[3, :32] = np.float32(np.nan)
    flags = mx.MX_FLAG_SCALE_CEIL if ceil else 0
    out = _quant(to_gpu_f32(x), 4, flags=flags)
    c, s, _ = host(out)
    wc, ws, _ = oracle.quantize(x, 4, variant=oracle.V_CEIL if ceil else 0)
    _same(s, ws, "scales")
    _same(c, wc, "codes")
    assert s[0, 0] == 254 and s[3, 0] == 0xFF


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_dequantize_bit_exact(fmt, rht, ydt):
    rows, cols = 96, 640
    x = W.normal_bf16(rows, cols, 2.0, fmt, 82, outlier_entries=0.01, outlier_mult=30.0)
    mask = oracle.rht_signs(fmt + 10)
    c, s, _ = oracle.quantize(x, fmt, rht=rht, sign_mask=mask)
    want = oracle.dequantize(fmt, c, s, None, rows, cols)
    if rht:
        want = oracle.rht16(want, mask, inverse=True)
    t = upload(fmt, c, s)
    t.cols = cols  # upload infers cols from the 8-bit or 4-bit code width
    y = torch.empty(rows, cols, dtype=torch.float32 if ydt == "f32" else torch.bfloat16, device=dev())
    mx.mx_dequantize(t, y, mx.MX_FLAG_RHT16 if rht else 0, mask)
    torch.cuda.synchronize()
    if ydt == "f32":
        _same(y.cpu().numpy().view(np.uint32), want.view(np.uint32), "decoded values")
    else:
        wb = W.f64_to_bf16_bits(want.astype(np.float64))
        _same(y.view(torch.int16).cpu().numpy().view(np.uint16), wb, "decoded bf16 values")


def test_s2f6_codec_round_trip_exact_on_representable_values():
    """Transformed values that are multiples of 2^-6 below 2, with every block
    maximum at least 1: encode (Hadamard + INT8) and decode (INT8 + inverse)
    return x bit for bit on the GPU too."""
    g = np.random.default_rng(13)
    mask = oracle.rht_signs(21)
    k = g.integers(-127, 128, (64, 1024))
    k[:, ::32] = -127  # block max 127/64 < 2: scale 2^0
    y = (k / 64.0).astype(np.float32)
    x = oracle.rht16(y, mask, inverse=True)
    out = _quant(to_gpu_f32(x), 4, flags=mx.MX_FLAG_RHT16, mask=mask)
    back = torch.empty(64, 1024, dtype=torch.float32, device=dev())
    mx.mx_dequantize(out, back, mx.MX_FLAG_RHT16, mask)
    torch.cuda.synchronize()
    _same(back.cpu().numpy().view(np.uint32), x.view(np.uint32), "round trip")


def test_s2f6_codec_moe_combine_size_sampled_rows():
    """The combine tensor of the MoE workload (32768 routed rows x 7168, BF16
    N(0,1)): Hadamard + INT8 encode on the GPU, checked against the oracle on
    bands of rows (rows are independent), and the decoded round trip's error
    against its bound: at most one step 2^(e-6) per transformed element (half
    a step when rounded, a full one when saturated at 127/64), carried over
    unchanged by the orthonormal inverse transform."""
    rows, cols = 32768, 7168
    bits = W.normal_bf16(rows, cols, 1.0, 0, 83)
    x = to_gpu_bf16(bits)
    mask = mx.mx_rht_signs(0)
    out = _quant(x, 4, flags=mx.MX_FLAG_RHT16, mask=mask)
    back = torch.empty(rows, cols, dtype=torch.float32, device=dev())
    mx.mx_dequantize(out, back, mx.MX_FLAG_RHT16, mask)
    torch.cuda.synchronize()
    c, s = out.codes.cpu().numpy(), out.scales.cpu().numpy()
    for r0 in (0, 12345, rows - 96):
        wc, ws, _ = oracle.quantize(bits[r0:r0 + 96], 4, rht=True, sign_mask=mask)
        _same(s[r0:r0 + 96], ws, f"scales rows {r0}..")
        _same(c[r0:r0 + 96], wc, f"codes rows {r0}..")
    xr = W.bf16_bits_to_f32(bits[:2048]).astype(np.float64)
    err = back[:2048].cpu().numpy().astype(np.float64) - xr
    # per 16-group: the transform is orthonormal, so the group's error norm is
    # the transformed error norm, each element of which is at most one step
    step = np.repeat(2.0 ** (s[:2048].astype(np.float64) - 127 - 6), 32, axis=1)
    gerr = np.sqrt((err ** 2).reshape(2048, -1, 16).sum(axis=2))
    gbound = np.sqrt((step ** 2).reshape(2048, -1, 16).sum(axis=2)) * (1 + 1e-5) + 1e-6
    assert np.all(gerr <= gbound)
    assert float(np.sqrt(np.mean(err ** 2))) < 0.015  # about step / sqrt(12) = 0.009 here


def test_other_formats_are_rejected_where_not_offered():
    """A pair with NVFP4, the FP8 flag on a non-FP8 pair, and the tile layout."""
    a = mx.empty(5, 64, 1024, device=dev())
    nv = mx.empty(3, 64, 1024, device=dev())
    C = torch.empty(64, 64, dtype=torch.float32, device=dev())
    with pytest.raises(mx.MXError):
        mx.mx_gemm(a, nv, C)
    i8 = mx.empty(4, 64, 1024, device=dev())
    with pytest.raises(mx.MXError):
        mx.mx_gemm_ex(i8, i8, C, mx.MX_GEMM_FP8_NATIVE)  # the FP8 instruction takes FP8 only
    tiled_fp6 = mx.empty(6, 64, 1024, device=dev(), layout=mx.MX_LAYOUT_TILED)
    with pytest.raises(mx.MXError):
        mx.mx_quantize(torch.zeros(64, 1024, dtype=torch.bfloat16, device=dev()), tiled_fp6)


# --- products of any pair of MX formats ---------------------------------------
ALL_MX = [1, 2, 4, 5, 6, 7]


def _operand(fmt, rows, K, seed, tid, std):
    x = W.normal_bf16(rows, K, std, seed, tid, outlier_entries=0.005, outlier_mult=20.0)
    c, s, _ = oracle.quantize(x, fmt)
    return c, s


@pytest.mark.parametrize("fa", ALL_MX)
@pytest.mark.parametrize("fb", ALL_MX)
def test_gemm_any_pair_of_mx_formats(fa, fb):
    """C = A * B^T with A and B in any MX formats (mixed included): exact
    products of the decoded operands, FP32 accumulation, within
    1e-5 * sum|a*b| of the oracle's FP64 product."""
    M, N, K = 200, 136, 320
    ca, sa = _operand(fa, M, K, fa * 10 + fb, 90, 1.0)
    cb, sb = _operand(fb, N, K, fa * 10 + fb, 91, 0.05)
    A = upload(fa, ca, sa)
    A.cols = K
    B = upload(fb, cb, sb)
    B.cols = K
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    if fa == fb and fa in (1, 2):
        pytest.skip("same-format MXFP8 / MXFP4 products have their own kernels and tests")
    mx.mx_gemm(A, B, C)
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(fa, ca, sa, M, K), oracle.dequantize_f64(fb, cb, sb, N, K))
    from tests.gpu_util import check_gemm
    check_gemm(C.cpu().numpy(), Cw, tol, False, f"fa={fa} fb={fb}")


@pytest.mark.parametrize("shape", [(1, 1, 32), (257, 129, 96), (512, 640, 2048)])
@pytest.mark.parametrize("cdt", ["f32", "bf16"])
def test_gemm_any_ragged_shapes_and_bf16_output(shape, cdt):
    M, N, K = shape
    ca, sa = _operand(4, M, K, 5, 92, 1.0)       # MXINT8 activations
    cb, sb = _operand(6, N, K, 5, 93, 0.05)      # MXFP6 E3M2 weights
    A = upload(4, ca, sa)
    A.cols = K
    B = upload(6, cb, sb)
    B.cols = K
    C = torch.empty(M, N, dtype=torch.float32 if cdt == "f32" else torch.bfloat16, device=dev())
    mx.mx_gemm(A, B, C)
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(4, ca, sa, M, K), oracle.dequantize_f64(6, cb, sb, N, K))
    from tests.gpu_util import check_gemm
    check_gemm(C.float().cpu().numpy(), Cw, tol, cdt == "bf16", f"{shape} {cdt}")


# --- E5M2 in the tile layout and on the scaled FP8 instruction -------------------
@pytest.mark.parametrize("rnd", [0, 1])
def test_e5m2_tiled_quantize_and_decode(rnd):
    from tests.tiles import untile_codes, untile_scales
    R, C = 64, 2048
    x = W.normal_bf16(R, C, 1.0, 4, 95, outlier_entries=0.002, outlier_mult=60)
    xt = to_gpu_bf16(x)
    out = mx.empty(5, R, C, device=dev(), layout=mx.MX_LAYOUT_TILED)
    mx.mx_quantize(xt, out, rnd, 3, 17)
    rows = mx.empty(5, R, C, device=dev())
    mx.mx_quantize(xt, rows, rnd, 3, 17)
    yt = torch.empty(R, C, dtype=torch.float32, device=dev())
    yr = torch.empty(R, C, dtype=torch.float32, device=dev())
    mx.mx_dequantize(out, yt)
    mx.mx_dequantize(rows, yr)
    torch.cuda.synchronize()
    c, s, _ = host(out)
    wc, ws, _ = oracle.quantize(x, 5, rnd, 3, 17)
    _same(untile_scales(s, R, C // 32), ws, "scales")
    _same(untile_codes(c, R, C), wc, "codes")
    assert torch.equal(yt.view(torch.int32), yr.view(torch.int32))


@pytest.mark.parametrize("fa,fb", [(5, 5), (5, 1), (1, 5)])
@pytest.mark.parametrize("cdt", ["f32", "bf16"])
def test_e5m2_pairs_on_the_fp8_instruction(fa, fb, cdt):
    """Tiled E4M3 / E5M2 pairs with MX_GEMM_FP8_NATIVE: within that flag's
    bound (1e-3 * sum|a*b|) of the oracle's exact product."""
    from tests.gpu_util import check_gemm
    from tests.tiles import tile_codes, tile_scales
    M, N, K = 288, 320, 2048
    ca, sa = _operand(fa, M, K, fa + 2 * fb, 96, 1.0)
    cb, sb = _operand(fb, N, K, fa + 2 * fb, 97, 0.05)
    A = mx.MXTensor(fa, M, K, torch.from_numpy(tile_codes(ca)).to(dev()), torch.from_numpy(tile_scales(sa)).to(dev()),
                    None, mx.MX_LAYOUT_TILED)
    B = mx.MXTensor(fb, N, K, torch.from_numpy(tile_codes(cb)).to(dev()), torch.from_numpy(tile_scales(sb)).to(dev()),
                    None, mx.MX_LAYOUT_TILED)
    C = torch.empty(M, N, dtype=torch.float32 if cdt == "f32" else torch.bfloat16, device=dev())
    with pytest.raises(mx.MXError):
        mx.mx_gemm(A, B, C)  # the FP8 instruction only on request
    mx.mx_gemm_ex(A, B, C, mx.MX_GEMM_FP8_NATIVE)
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(fa, ca, sa, M, K), oracle.dequantize_f64(fb, cb, sb, N, K))
    check_gemm(C.float().cpu().numpy(), Cw, tol * 100, cdt == "bf16", f"fa={fa} fb={fb} {cdt}")


def test_e5m2_tiled_jobs_in_a_batch():
    T = mx.MX_LAYOUT_TILED
    xs = [to_gpu_bf16(W.normal_bf16(64, 1024, 1.0, 40 + i, 98)) for i in range(3)]
    outs = [mx.empty(5, 64, 1024, device=dev(), layout=T) for _ in xs]
    mx.mx_quantize_batch([dict(x=x, out=o, rnd=1, seed=9, counter=100 * i) for i, (x, o) in enumerate(zip(xs, outs))])
    singles = [mx.empty(5, 64, 1024, device=dev(), layout=T) for _ in xs]
    for i, (x, o) in enumerate(zip(xs, singles)):
        mx.mx_quantize(x, o, 1, 9, 100 * i)
    torch.cuda.synchronize()
    for o, s1 in zip(outs, singles):
        assert torch.equal(o.codes, s1.codes) and torch.equal(o.scales, s1.scales)


# --- FP6 pairs on the scaled FP6/FP4 matrix instruction ----------------------------
F6_PAIRS = [(7, 7), (7, 6), (6, 7), (7, 2), (2, 7), (6, 2), (2, 6), (6, 6)]


def _operand_blocks(fmt, rows, K, seed, tid, std):
    """Rows and K-blocks scaled by independent powers of two (2^-12 .. 2^12), so
    that the scale codes of a row's blocks differ and a block scale applied to
    the wrong block or lane group shows."""
    x = W.bf16_bits_to_f32(W.normal_bf16(rows, K, std, seed, tid)).astype(np.float64)
    g = W.rng(seed, tid + 1)
    x *= np.exp2(g.integers(-12, 13, (rows, 1)))
    x *= np.repeat(np.exp2(g.integers(-12, 13, (1, K // 32))), 32, axis=1)
    c, s, _ = oracle.quantize(W.f64_to_bf16_bits(x), fmt)
    return c, s


@pytest.mark.parametrize("fa,fb", F6_PAIRS)
@pytest.mark.parametrize("shape", [(200, 136, 384), (300, 520, 1024), (33, 257, 128), (520, 300, 2560)])
def test_gemm_fp6_pairs_on_the_scaled_instruction(fa, fb, shape):
    """K % 512 == 0: the FP6 pairs run on the scaled FP6/FP4 instruction (E3M2 x
    E3M2 on the BF16 kernel), within 1e-5 * sum|a*b| of the oracle's FP64
    product; ragged M and N, several workgroup tiles, 8 and 20 K steps (2 and
    5 scale periods).  K = 384 and 128 take the BF16 kernel for every pair."""
    M, N, K = shape
    seed = fa * 10 + fb + K
    ca, sa = _operand_blocks(fa, M, K, seed, 94, 1.0)
    cb, sb = _operand_blocks(fb, N, K, seed, 96, 0.05)
    A = upload(fa, ca, sa)
    A.cols = K
    B = upload(fb, cb, sb)
    B.cols = K
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm(A, B, C)
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(fa, ca, sa, M, K), oracle.dequantize_f64(fb, cb, sb, N, K))
    from tests.gpu_util import check_gemm
    check_gemm(C.cpu().numpy(), Cw, tol, False, f"fa={fa} fb={fb} {shape}")


@pytest.mark.parametrize("fa,fb", [(7, 2), (6, 7)])
def test_gemm_fp6_bf16_output_and_strided_c(fa, fb):
    """BF16 output into a C with a row pitch wider than N (element stores)."""
    M, N, K, ldc = 160, 200, 512, 264
    ca, sa = _operand_blocks(fa, M, K, 3, 98, 1.0)
    cb, sb = _operand_blocks(fb, N, K, 3, 100, 0.05)
    A = upload(fa, ca, sa)
    A.cols = K
    B = upload(fb, cb, sb)
    B.cols = K
    Cbuf = torch.full((M, ldc), 7.0, dtype=torch.bfloat16, device=dev())
    mx.mx_gemm(A, B, Cbuf[:, :N])
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(fa, ca, sa, M, K), oracle.dequantize_f64(fb, cb, sb, N, K))
    from tests.gpu_util import check_gemm
    got = Cbuf.float().cpu().numpy()
    check_gemm(got[:, :N], Cw, tol, True, f"fa={fa} fb={fb} bf16")
    assert np.all(got[:, N:] == 7.0)


def test_gemm_fp6_full_size_sampled():
    """4096^3 MXFP6 E2M3 x MXFP4 (the launch the benchmark times), checked on
    sampled rows and columns against the oracle's exact product."""
    M = N = K = 4096
    ca, sa = _operand(7, M, K, 1, 102, 1.0)
    cb, sb = _operand(2, N, K, 1, 104, 0.05)
    A = upload(7, ca, sa)
    A.cols = K
    B = upload(2, cb, sb)
    B.cols = K
    C = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    mx.mx_gemm(A, B, C)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    ri = g.integers(0, M, 3000)
    cj = g.integers(0, N, 3000)
    Cw, tol = oracle.gemm_sampled(oracle.dequantize_f64(7, ca, sa, M, K), oracle.dequantize_f64(2, cb, sb, N, K),
                                  ri, cj)
    from tests.gpu_util import check_gemm
    got = C.float().cpu().numpy()[ri, cj]
    check_gemm(got, Cw, tol, True, "4096^3 e2m3 x e2m1")


@pytest.mark.parametrize("fa,fb,csum", [(7, 7, 135), (6, 7, 135), (7, 2, 135), (2, 6, 135), (2, 2, 130)])
def test_scaled_instruction_at_the_low_scale_limit(fa, fb, csum):
    """The scaled matrix instructions flush FP32-subnormal partial sums; the
    bound holds while c_A + c_B reaches the documented limit, where the
    smallest nonzero product is exactly 2^-126 or above (random codes, every
    block of A at scale code c_A and of B at c_B)."""
    M, N, K = 96, 160, 512
    g = np.random.default_rng(csum + fa + fb)
    def codes(fmt, rows):
        bits = 8 if fmt in (1, 4, 5) else 6 if fmt in (6, 7) else 4
        c, _, _ = oracle.quantize(np.zeros((rows, K), np.uint16), fmt)
        raw = g.integers(0, 1 << bits, (rows, K))
        packed = np.zeros_like(c)
        for k in range(K):  # element k at bits bits*k of the row
            bit = bits * k
            packed[:, bit // 8] |= ((raw[:, k] << (bit % 8)) & 0xFF).astype(np.uint8)
            if bit % 8 + bits > 8:
                packed[:, bit // 8 + 1] |= (raw[:, k] >> (8 - bit % 8)).astype(np.uint8)
        return packed
    ca, cb = codes(fa, M), codes(fb, N)
    sa = np.full((M, K // 32), csum // 2, np.uint8)
    sb = np.full((N, K // 32), csum - csum // 2, np.uint8)
    A = upload(fa, ca, sa)
    A.cols = K
    B = upload(fb, cb, sb)
    B.cols = K
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm(A, B, C)
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(fa, ca, sa, M, K), oracle.dequantize_f64(fb, cb, sb, N, K))
    from tests.gpu_util import check_gemm
    check_gemm(C.cpu().numpy(), Cw, tol, False, f"fa={fa} fb={fb} c_A+c_B={csum}")
    assert np.abs(Cw).max() < 2.0**-100  # the products really are tiny


@pytest.mark.parametrize("fa,fb,K", [(5, 1, 512), (1, 5, 512), (5, 5, 512), (5, 1, 2048), (4, 4, 512),
                                     (4, 4, 2048), (4, 1, 512), (1, 4, 512), (4, 5, 512), (5, 4, 512)])
@pytest.mark.parametrize("cdt", ["f32", "bf16"])
def test_8bit_pairs_on_the_exact_pipeline(fa, fb, K, cdt):
    """Pairs of 8-bit MX types (E4M3, E5M2, INT8) other than E4M3 x E4M3, at a
    size the exact 8-bit pipeline takes (BF16 instruction, 1e-5 bound), with scale codes 0 and 255
    in a few blocks of A and B: the fix-up pass recomputes those tiles, NaN
    reaches exactly the rows and columns the oracle gives, everything else
    stays in the bound."""
    M, N = 2048, 4096
    ca, sa = _operand(fa, M, K, 10 * fa + fb, 106, 1.0)
    cb, sb = _operand(fb, N, K, 10 * fa + fb, 108, 0.05)
    sa, sb = sa.copy(), sb.copy()
    sa[5, 3] = 0
    sa[700, 10] = 255
    sb[1234, 7] = 0
    sb[3000, 2] = 255
    A = upload(fa, ca, sa)
    A.cols = K
    B = upload(fb, cb, sb)
    B.cols = K
    dt = torch.float32 if cdt == "f32" else torch.bfloat16
    C = torch.full((M, N), 7.0, dtype=dt, device=dev())
    mx.mx_gemm(A, B, C)
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(fa, ca, sa, M, K), oracle.dequantize_f64(fb, cb, sb, N, K))
    got = C.float().cpu().numpy()
    nan_want = np.isnan(Cw)
    assert nan_want[700].all() and nan_want[:, 3000].all() and nan_want.sum() == N + M - 1
    assert np.isnan(got[nan_want]).all(), "NaN scale blocks must give NaN outputs"
    keep = ~nan_want
    assert not np.isnan(got[keep]).any()
    from tests.gpu_util import check_gemm
    check_gemm(np.where(keep, got, 0.0), np.where(keep, Cw, 0.0), np.where(keep, tol, 1.0), cdt == "bf16",
               f"fa={fa} fb={fb} {cdt}")


@pytest.mark.parametrize("fa,fb", [(5, 1), (1, 5), (5, 5)])
@pytest.mark.parametrize("shape", [(288, 320, 2048), (2048, 4096, 512)])
def test_e5m2_row_layout_pairs_on_the_fp8_instruction(fa, fb, shape):
    """Row-layout FP8 pairs with E5M2 and MX_GEMM_FP8_NATIVE (the small-shape
    kernel and the DMA pipeline): within that flag's bound (1e-3 * sum|a*b|)."""
    from tests.gpu_util import check_gemm
    M, N, K = shape
    ca, sa = _operand(fa, M, K, fa + 3 * fb, 110, 1.0)
    cb, sb = _operand(fb, N, K, fa + 3 * fb, 111, 0.05)
    A = upload(fa, ca, sa)
    A.cols = K
    B = upload(fb, cb, sb)
    B.cols = K
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm_ex(A, B, C, mx.MX_GEMM_FP8_NATIVE)
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(fa, ca, sa, M, K), oracle.dequantize_f64(fb, cb, sb, N, K))
    check_gemm(C.cpu().numpy(), Cw, tol * 100, False, f"fa={fa} fb={fb} {shape}")


@pytest.mark.parametrize("cdt", ["f32", "bf16"])
def test_e3m2_pair_decoded_with_special_scale_codes(cdt):
    """E3M2 x E3M2 (K % 512 == 0) is decoded to BF16 inside the FP6 kernel;
    tiles whose operands hold scale code 0 or 255 are recomputed by the
    generic kernel's fix-up pass: NaN exactly where the oracle has it, the
    rest within the bound."""
    M, N, K = 300, 520, 1024
    ca, sa = _operand_blocks(6, M, K, 77, 112, 1.0)
    cb, sb = _operand_blocks(6, N, K, 77, 114, 0.05)
    sa, sb = sa.copy(), sb.copy()
    sa[5, 3] = 0
    sa[200, 10] = 255
    sb[130, 7] = 0
    sb[400, 2] = 255
    A = upload(6, ca, sa)
    A.cols = K
    B = upload(6, cb, sb)
    B.cols = K
    C = torch.full((M, N), 7.0, dtype=torch.float32 if cdt == "f32" else torch.bfloat16, device=dev())
    mx.mx_gemm(A, B, C)
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(6, ca, sa, M, K), oracle.dequantize_f64(6, cb, sb, N, K))
    got = C.float().cpu().numpy()
    nan_want = np.isnan(Cw)
    assert nan_want[200].all() and nan_want[:, 400].all()
    assert np.isnan(got[nan_want]).all()
    keep = ~nan_want
    assert not np.isnan(got[keep]).any()
    from tests.gpu_util import check_gemm
    check_gemm(np.where(keep, got, 0.0), np.where(keep, Cw, 0.0), np.where(keep, tol, 1.0), cdt == "bf16",
               f"e3m2 pair {cdt}")
