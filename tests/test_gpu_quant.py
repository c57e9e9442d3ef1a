"""GPU parity of the quantizers, amax, decoder, Hadamard transform and
requant-transpose against the CPU oracle: bit-exact codes, scales and tensor
scales (SR included, same seed and counter), on shapes that span several
workgroups and ragged tails, both input dtypes and strided inputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import (bf16_bits_of, dev, host, quantize_gpu, to_gpu_bf16, to_gpu_f32,
                                upload)

SHAPES = [(1, 32), (7, 96), (33, 256), (130, 544), (257, 1024)]


def _inputs(rows, cols, dt, seed, pad=0):
    bits = W.normal_bf16(rows, cols, 1.5, seed, 40, outlier_entries=0.01, outlier_mult=60.0)
    if dt == "bf16":
        return bits, to_gpu_bf16(bits, pad)
    f = W.bf16_bits_to_f32(bits) * np.float32(1.0 + 2.0**-12)  # full FP32 mantissas
    f = f.astype(np.float32)
    return f, to_gpu_f32(f, pad)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_mx_quantize_bit_exact(shape, fmt, rnd, rht, dt):
    rows, cols = shape
    seed = rows * 31 + cols + fmt * 7 + rnd
    x_np, x = _inputs(rows, cols, dt, seed, pad=16 if rows % 2 else 0)
    mask = oracle.rht_signs(seed)
    out, _ = quantize_gpu(x, fmt, rnd, seed=seed, counter=3 * seed + 1, rht=rht, mask=mask)
    c, s, _ = host(out)
    wc, ws, _ = oracle.quantize(x_np, fmt, rnd, seed=seed, counter=3 * seed + 1, rht=rht,
                                sign_mask=mask)
    assert np.array_equal(s, ws), f"scales differ at {np.argwhere(s != ws)[:5]}"
    assert np.array_equal(c, wc), f"codes differ at {np.argwhere(c != wc)[:5]}"


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_nvfp4_quantize_bit_exact(shape, rnd, rht, dt):
    rows, cols = shape
    seed = rows * 17 + cols + rnd
    x_np, x = _inputs(rows, cols, dt, seed, pad=8 if rows % 2 else 0)
    mask = oracle.rht_signs(seed + 1)
    out, amax = quantize_gpu(x, 3, rnd, seed=seed, counter=5, rht=rht, mask=mask)
    c, s, ts = host(out)
    wc, ws, wts = oracle.quantize(x_np, 3, rnd, seed=seed, counter=5, rht=rht, sign_mask=mask)
    assert float(amax.cpu()[0]) == oracle.tensor_amax(x_np, rht, mask)
    assert float(ts[0]) == wts
    assert np.array_equal(s, ws), f"scales differ at {np.argwhere(s != ws)[:5]}"
    assert np.array_equal(c, wc), f"codes differ at {np.argwhere(c != wc)[:5]}"


@pytest.mark.parametrize("shape", [(1, 16), (1, 48), (3, 16), (5, 80)])
def test_amax_with_hadamard_on_tensors_shorter_than_a_wave(shape):
    """Fewer chunks than lanes: lanes past the end must not add transformed
    duplicates of the last chunk to the maximum."""
    rows, cols = shape
    bits = W.normal_bf16(rows, cols, 1.0, rows + cols, 42)
    mask = oracle.rht_signs(rows * cols)
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    mx.mx_amax(to_gpu_bf16(bits), amax, mx.MX_FLAG_RHT16, mask)
    torch.cuda.synchronize()
    assert float(amax.cpu()[0]) == oracle.tensor_amax(bits, True, mask)


def test_nvfp4_amax_given_and_zero_tensor():
    bits = W.normal_bf16(64, 128, 1.0, 3, 41)
    x = to_gpu_bf16(bits)
    out, _ = quantize_gpu(x, 3, 0, amax_value=7.25)
    c, s, ts = host(out)
    wc, ws, wts = oracle.quantize(bits, 3, amax=7.25)
    assert float(ts[0]) == wts and np.array_equal(c, wc) and np.array_equal(s, ws)
    z = torch.zeros(16, 64, dtype=torch.bfloat16, device=dev())
    z[3, 5] = -0.0
    out, amax = quantize_gpu(z, 3, 1)
    c, s, ts = host(out)
    wc, ws, wts = oracle.quantize(bf16_bits_of(z), 3, 1)
    assert float(ts[0]) == 1.0 == wts and np.array_equal(c, wc) and np.array_equal(s, ws)


@pytest.mark.parametrize("t_exp", [-137, -126, -81, -80, -72, -70, 0, 88, 89, 90, 127])
def test_nvfp4_given_amax_across_the_divisor_range(t_exp):
    """A given tensor amax T = 1.75 * 2^t_exp puts the block-scale divisor
    d = 6 fl(T / 2688) on both sides of the range where the quotient is
    formed as a corrected product (2^-80 <= d <= 2^80) and at the FP32
    extremes, with subnormal T, reciprocals that overflow to +Inf and blocks
    whose maximum lies far below T, at T and (below the FP32 limit) above it.
    Codes, block scales and the tensor scale match the oracle bit for bit for
    the 1-D, 2-D and Four Over Six encoders."""
    T = np.float32(1.75) * np.float32(2.0) ** np.float32(t_exp)
    assert np.isfinite(T) and T > 0
    rows, cols = 48, 256
    rng = np.random.default_rng(t_exp + 200)
    u = rng.uniform(-1.0, 1.0, size=(rows, cols))
    shrink = 2.0 ** rng.integers(0, 40, size=(rows, cols // 16))  # per block: 2^0 .. 2^-39 of T
    u = u / np.repeat(shrink, 16, axis=1)
    if t_exp < 100:
        u[::5, 3] = 1.5  # blocks above the given amax: their scale saturates
    x = (u * np.float64(T)).astype(np.float32)
    assert np.all(np.isfinite(x))
    xd = to_gpu_f32(x)
    for flags, rnd in ((0, 0), (0, 1), (mx.MX_FLAG_BLOCK_2D, 0), (mx.MX_FLAG_BLOCK_2D, 1),
                       (mx.MX_FLAG_FOUR_OVER_SIX, 0)):
        out = mx.empty(3, rows, cols, device=dev())
        amax = torch.full((1,), float(T), dtype=torch.float32, device=dev())
        mx.mx_quantize(xd, out, rnd, 5, 9, flags | mx.MX_FLAG_AMAX_GIVEN, 0, amax)
        torch.cuda.synchronize()
        c, s, ts = host(out)
        variant = oracle.V_2D if flags == mx.MX_FLAG_BLOCK_2D else (
            oracle.V_FOUR6 if flags == mx.MX_FLAG_FOUR_OVER_SIX else 0)
        wc, ws, wts = oracle.quantize(x, 3, rnd, seed=5, counter=9, amax=float(T), variant=variant)
        assert float(ts[0]) == wts, (t_exp, flags, rnd)
        assert np.array_equal(s, ws), (t_exp, flags, rnd, np.argwhere(s != ws)[:5])
        assert np.array_equal(c, wc), (t_exp, flags, rnd, np.argwhere(c != wc)[:5])


def test_mx_special_values():
    """All-zero blocks, signed zeros, NaN/Inf blocks, FP32 subnormals, values
    at the saturation limits and exact ties."""
    x = np.zeros((4, 128), np.float32)
    x[0, 1] = -0.0
    x[1, 0:32] = np.float32(1e-40) * np.arange(32)         # subnormal block
    x[1, 40] = np.inf
    x[1, 64:96] = np.linspace(-500, 500, 32)                # saturating E4M3 after scaling
    x[2, 0:32] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4   # E2M1 ties (scale 2^0)
    x[2, 32] = np.nan
    x[3, :] = np.float32(3.0e38) * np.sin(np.arange(128))   # near FP32 max
    for fmt in (1, 2):
        for rnd in (0, 1):
            out, _ = quantize_gpu(to_gpu_f32(x), fmt, rnd, seed=9)
            c, s, _ = host(out)
            wc, ws, _ = oracle.quantize(x, fmt, rnd, seed=9)
            assert np.array_equal(s, ws) and np.array_equal(c, wc), (fmt, rnd)


def test_sr_determinism_and_counter():
    bits = W.normal_bf16(96, 512, 1.0, 4, 42)
    x = to_gpu_bf16(bits)
    a, _ = quantize_gpu(x, 2, 1, seed=11, counter=100)
    b, _ = quantize_gpu(x, 2, 1, seed=11, counter=100)
    c, _ = quantize_gpu(x, 2, 1, seed=11, counter=101)
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    assert not torch.equal(a.codes, c.codes)


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
@pytest.mark.parametrize("rht", [False, True])
def test_dequantize(fmt, ydt, rht):
    rows, cols = 70, 352
    bits = W.normal_bf16(rows, cols, 2.0, 5, 43, outlier_entries=0.02, outlier_mult=40)
    mask = oracle.rht_signs(7)
    wc, ws, wts = oracle.quantize(bits, fmt, 0)
    t = upload(fmt, wc, ws, wts)
    y = torch.empty(rows, cols, dtype=torch.float32 if ydt == "f32" else torch.bfloat16, device=dev())
    mx.mx_dequantize(t, y, mx.MX_FLAG_RHT16 if rht else 0, mask)
    torch.cuda.synchronize()
    want = oracle.dequantize(fmt, wc, ws, wts, rows, cols)
    if rht:
        want = oracle.rht16(want, mask, inverse=True)
    if ydt == "f32":
        assert np.array_equal(y.cpu().numpy(), want)
    else:
        assert np.array_equal(bf16_bits_of(y), W.f64_to_bf16_bits(want.astype(np.float64)))


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("ydt", ["bf16", "f32"])
@pytest.mark.parametrize("inverse", [False, True])
def test_hadamard16(xdt, ydt, inverse):
    rows, cols = 45, 208
    bits = W.normal_bf16(rows, cols, 3.0, 6, 44)
    mask = oracle.rht_signs(8)
    if xdt == "bf16":
        x, xin = to_gpu_bf16(bits).contiguous(), bits
    else:
        f = W.bf16_bits_to_f32(bits) * np.float32(1.0 + 2.0**-13)
        x, xin = to_gpu_f32(f.astype(np.float32)).contiguous(), f.astype(np.float32)
    y = torch.empty(rows, cols, dtype=torch.float32 if ydt == "f32" else torch.bfloat16, device=dev())
    mx.mx_hadamard16(x, y, mask, inverse)
    torch.cuda.synchronize()
    want = oracle.rht16(xin, mask, inverse)
    if ydt == "f32":
        assert np.array_equal(y.cpu().numpy(), want)
    else:
        assert np.array_equal(bf16_bits_of(y), W.f64_to_bf16_bits(want.astype(np.float64)))


def test_hadamard16_in_place_roundtrip():
    x = torch.randn(64, 128, device=dev())
    ref = x.clone()
    mx.mx_hadamard16(x, x, 0x5A5A)
    mx.mx_hadamard16(x, x, 0x5A5A, inverse=True)
    torch.cuda.synchronize()
    assert torch.allclose(x, ref, atol=1e-6, rtol=1e-6)


@pytest.mark.parametrize("shape", [(32, 16), (64, 256), (96, 48), (160, 272), (320, 528)])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("src", ["nvfp4", "bf16"])
def test_requant_transpose_bit_exact(shape, rnd, src):
    rows, cols = shape
    bits = W.normal_bf16(rows, cols, 1.0, rows + cols, 45, outlier_entries=0.005, outlier_mult=30)
    out = mx.empty(1, cols, rows, device=dev())
    if src == "nvfp4":
        nv = oracle.quantize(bits, 3, 0)
        t = upload(3, nv[0], nv[1], nv[2])
        mx.mx_requant_transpose(out, src=t, rnd=rnd, seed=13, counter=rows)
        wc, ws = oracle.requant_transpose(rows, cols, rnd, seed=13, counter=rows, nvfp4=nv)
    else:
        x = to_gpu_bf16(bits, pad_cols=8)
        mx.mx_requant_transpose(out, x_bf16=x, rnd=rnd, seed=13, counter=rows)
        wc, ws = oracle.requant_transpose(rows, cols, rnd, seed=13, counter=rows, bf16=bits)
    torch.cuda.synchronize()
    c, s, _ = host(out)
    assert np.array_equal(s, ws), f"scales differ at {np.argwhere(s != ws)[:5]}"
    assert np.array_equal(c, wc), f"codes differ at {np.argwhere(c != wc)[:5]}"


@pytest.mark.parametrize("ts", [2.0 ** -120, 2.0 ** -116, 2.0 ** -100, 0.0, 1e38, float("inf"), float("nan")])
@pytest.mark.parametrize("rnd", [0, 1])
def test_requant_transpose_tensor_scale_edges(ts, rnd):
    """NVFP4 source whose tensor scale makes p * S subnormal, zero, overflow
    or NaN, with all-zero blocks in the first 64 rows."""
    rows, cols = 256, 192
    bits = W.normal_bf16(rows, cols, 1.0, 7, 47)
    nv = oracle.quantize(bits, 3, 0)
    codes = nv[0].copy()
    codes[:64] = 0
    tsv = np.float32(ts)
    out = mx.empty(1, cols, rows, device=dev())
    mx.mx_requant_transpose(out, src=upload(3, codes, nv[1], tsv), rnd=rnd, seed=5, counter=3)
    wc, ws = oracle.requant_transpose(rows, cols, rnd, seed=5, counter=3, nvfp4=(codes, nv[1], tsv))
    torch.cuda.synchronize()
    c, s, _ = host(out)
    assert np.array_equal(s, ws), f"scales differ at {np.argwhere(s != ws)[:5]}"
    assert np.array_equal(c, wc), f"codes differ at {np.argwhere(c != wc)[:5]}"


@pytest.mark.parametrize("shape", [(256, 320), (224, 336)])
@pytest.mark.parametrize("rnd", [0, 1])
def test_requant_transpose_every_e4m3_scale_code(shape, rnd):
    """NVFP4 source with random FP4 codes and block scales drawn from every
    finite E4M3 code 0..126 (subnormal scales included): the decode of each
    scale code against the oracle's."""
    rows, cols = shape
    rng = np.random.default_rng(rows + cols)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 127, size=(rows, cols // 16), dtype=np.uint8)
    scales.flat[:127] = np.arange(127, dtype=np.uint8)
    ts = np.float32(0.37)
    out = mx.empty(1, cols, rows, device=dev())
    mx.mx_requant_transpose(out, src=upload(3, codes, scales, ts), rnd=rnd, seed=2, counter=11)
    wc, ws = oracle.requant_transpose(rows, cols, rnd, seed=2, counter=11, nvfp4=(codes, scales, ts))
    torch.cuda.synchronize()
    c, s, _ = host(out)
    assert np.array_equal(s, ws), f"scales differ at {np.argwhere(s != ws)[:5]}"
    assert np.array_equal(c, wc), f"codes differ at {np.argwhere(c != wc)[:5]}"


def test_requant_transpose_nvfp4_several_tiles_per_workgroup():
    """4096 x 4096 NVFP4 source: 2048 tiles of 128 x 64, several per
    workgroup of the persistent grid; bit-exact against the oracle and
    identical over repeated launches (no LDS race between a workgroup's
    tiles or between its producer and consumer waves)."""
    rows, cols = 4096, 4096
    bits = W.normal_bf16(rows, cols, 1.0, 3, 48, outlier_entries=0.001, outlier_mult=20)
    nv = oracle.quantize(bits, 3, 0)
    t = upload(3, nv[0], nv[1], nv[2])
    ref = mx.empty(1, cols, rows, device=dev())
    mx.mx_requant_transpose(ref, src=t, rnd=1, seed=9, counter=77)
    wc, ws = oracle.requant_transpose(rows, cols, 1, seed=9, counter=77, nvfp4=nv)
    torch.cuda.synchronize()
    c, s, _ = host(ref)
    assert np.array_equal(s, ws), f"scales differ at {np.argwhere(s != ws)[:5]}"
    assert np.array_equal(c, wc), f"codes differ at {np.argwhere(c != wc)[:5]}"
    for _ in range(10):
        o = mx.empty(1, cols, rows, device=dev())
        mx.mx_requant_transpose(o, src=t, rnd=1, seed=9, counter=77)
        assert torch.equal(o.codes, ref.codes) and torch.equal(o.scales, ref.scales)


def test_requant_transpose_repeatable():
    """No LDS race: 20 repeated launches give identical bytes."""
    bits = W.normal_bf16(512, 1024, 1.0, 1, 46)
    x = to_gpu_bf16(bits)
    ref = mx.empty(1, 1024, 512, device=dev())
    mx.mx_requant_transpose(ref, x_bf16=x, rnd=1, seed=1)
    for _ in range(20):
        o = mx.empty(1, 1024, 512, device=dev())
        mx.mx_requant_transpose(o, x_bf16=x, rnd=1, seed=1)
        assert torch.equal(o.codes, ref.codes) and torch.equal(o.scales, ref.scales)
