"""GPU checks of the GEMM that quantizes its A operand in the prologue
(mx_gemm_quantize_a): Q(A), written out by the kernel, is bit for bit the
oracle's MX quantization of A (RNE and SR, the SR stream indexed by the
element's position in A); C = Q(A) * B^T is checked entry by entry against
the oracle's FP64 product of the decoded operands within the GEMM bound."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import check_gemm, dev, host, to_gpu_bf16, upload


def _run(M, N, K, a_fmt, b_fmt, rnd, cdt, seed=0, pad=0, nan_rows=(), emit=True, low_b_rows=()):
    A = W.normal_bf16(M, K, 1.0, M + N, 60, outlier_entries=0.002, outlier_mult=40.0)
    for r in nan_rows:
        A[r, 37] = 0x7FC0  # a NaN: its block gets scale 0xFF and zero codes
    Bb = W.normal_bf16(N, K, 0.05, M + N, 61)
    qb = oracle.quantize(Bb, b_fmt)
    for r in low_b_rows:  # scale codes whose products with Q(A)'s are subnormal FP32 values
        qb[1][r] = (20 if b_fmt == 1 else 2) + (np.arange(K // 32) % 7)
    B = upload(b_fmt, qb[0], qb[1])
    tdt = torch.float32 if cdt == 1 else torch.bfloat16
    C = torch.empty(M, N + 3, dtype=tdt, device=dev())[:, :N]
    qa = mx.empty(a_fmt, M, K, device=dev()) if emit else None
    mx.mx_gemm_quantize_a(to_gpu_bf16(A, pad_cols=pad), a_fmt, B, C, rnd, seed=seed, counter=M, a_out=qa)
    torch.cuda.synchronize()
    oa = oracle.quantize(A, a_fmt, rnd, seed=seed, counter=M)
    if emit:
        c, s, _ = host(qa)
        assert np.array_equal(s, oa[1]), f"scales differ at {np.argwhere(s != oa[1])[:5]}"
        assert np.array_equal(c, oa[0]), f"codes differ at {np.argwhere(c != oa[0])[:5]}"
    Chat, tol = oracle.gemm(oracle.dequantize_f64(a_fmt, oa[0], oa[1], M, K),
                            oracle.dequantize_f64(b_fmt, qb[0], qb[1], N, K))
    check_gemm(C.float().cpu().numpy(), Chat, tol, cdt == 0, f"qa {a_fmt}x{b_fmt} rnd {rnd}")
    return C


@pytest.mark.parametrize("a_fmt,b_fmt", [(1, 1), (2, 2), (1, 2), (2, 1)])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("shape", [(96, 160, 256), (130, 72, 1056)])
def test_prologue_quantized_gemm_small(a_fmt, b_fmt, rnd, shape):
    """Ragged 128x128-tile launches: partial row and column tiles, K not a
    multiple of the 64-element step, an A pitch wider than K."""
    M, N, K = shape
    _run(M, N, K, a_fmt, b_fmt, rnd, cdt=1, seed=3, pad=8)


@pytest.mark.parametrize("a_fmt,b_fmt", [(1, 1), (2, 2)])
@pytest.mark.parametrize("cdt", [0, 1])
def test_prologue_quantized_gemm_256_tiles(a_fmt, b_fmt, cdt):
    """2048 x 4096 x 512: the 256x256-tile launch; BF16 and FP32 output."""
    _run(2048, 4096, 512, a_fmt, b_fmt, 1, cdt, seed=5)


def test_prologue_quantized_gemm_nan_blocks_and_no_output_copy():
    """Rows whose block holds a NaN get scale 0xFF and NaN products in
    exactly those rows; without a_out the product is unchanged."""
    C1 = _run(64, 96, 128, 1, 1, 0, cdt=1, nan_rows=(3, 40))
    C2 = _run(64, 96, 128, 1, 1, 0, cdt=1, nan_rows=(3, 40), emit=False)
    assert torch.equal(torch.isnan(C1), torch.isnan(C2))
    c1, c2 = C1.nan_to_num(0.0), C2.nan_to_num(0.0)
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("a_fmt,b_fmt", [(1, 1), (2, 2), (2, 1)])
def test_prologue_quantized_gemm_low_b_codes_with_q_a_written(a_fmt, b_fmt):
    """Rows of B at scale codes 20 .. 26 (E4M3) or 2 .. 8 (E2M1), whose
    products with Q(A)'s blocks (codes near 120) are subnormal FP32 values:
    with Q(A) written out, the fix-up pass recomputes those tiles and every
    output is within the bound (FP32 out, checked in full)."""
    _run(384, 320, 1024, a_fmt, b_fmt, 0, cdt=1, seed=2, low_b_rows=(0, 77, 300))
