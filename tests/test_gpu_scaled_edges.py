"""Edge cases of the GEMMs on gfx950's scaled matrix instruction
(v_mfma_scale_f32_32x32x64_f8f6f4), against the CPU oracle:

* scale code 0xFF (E8M0 NaN, what the quantizers write for a block holding
  NaN or Inf): NaN exactly in the rows of A and columns of B the oracle gives,
  in the tile layout (MXFP4), the row layout (MXFP4) and for FP6 pairs;
* scale codes so small that products fall below FP32's subnormal spacing
  (c_A + c_B < 105 + g_A + g_B, e.g. 107 for FP4): whole rows and whole tiles
  of such codes, next to ordinary ones.  The instruction itself rounds once
  (subnormals included); a tile where such pairs can occur is computed again
  with raised codes and scaled back with one rounding, so the FP32 output is
  the rounding of a value within the bound.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import check_gemm, dev, upload
    from tests.tiles import tile_codes, tile_scales


def _bits(fmt):
    return 8 if fmt in (1, 4, 5) else 6 if fmt in (6, 7) else 4


def _codes(g, fmt, rows, K):
    """Random element codes of every value (row layout, packed)."""
    bits = _bits(fmt)
    raw = g.integers(0, 1 << bits, (rows, K))
    if bits == 8:
        if fmt == 1:  # no E4M3 NaN (S.1111.111)
            raw = np.where((raw & 0x7F) == 0x7F, raw & 0xF0, raw)
        if fmt == 5:  # no E5M2 Inf / NaN (exponent 11111)
            raw = np.where((raw & 0x7C) == 0x7C, raw & 0x83, raw)
        return raw.astype(np.uint8)
    if bits == 4:
        return (raw[:, 0::2] | (raw[:, 1::2] << 4)).astype(np.uint8)
    packed = np.zeros((rows, K * 6 // 8), np.uint8)
    for k in range(K):  # element k at bits 6k of the row
        bit = 6 * k
        packed[:, bit // 8] |= ((raw[:, k] << (bit % 8)) & 0xFF).astype(np.uint8)
        if bit % 8 + 6 > 8:
            packed[:, bit // 8 + 1] |= (raw[:, k] >> (8 - bit % 8)).astype(np.uint8)
    return packed


def _upload(fmt, codes, scales, tiled):
    R = codes.shape[0]
    K = scales.shape[1] * 32
    if tiled:
        return mx.MXTensor(fmt, R, K, torch.from_numpy(tile_codes(codes)).to(dev()),
                           torch.from_numpy(tile_scales(scales)).to(dev()), None, mx.MX_LAYOUT_TILED)
    t = upload(fmt, codes, scales)
    t.cols = K
    return t


def _run(fa, fb, ca, sa, cb, sb, M, N, K, tiled, cdt):
    A, B = _upload(fa, ca, sa, tiled), _upload(fb, cb, sb, tiled)
    C = torch.empty(M, N, dtype=torch.float32 if cdt == "f32" else torch.bfloat16, device=dev())
    if tiled and fa in (1, 5):  # FP8 on the tile layout: the native instruction only
        mx.mx_gemm_ex(A, B, C, mx.MX_GEMM_FP8_NATIVE)
    else:
        mx.mx_gemm(A, B, C)
    torch.cuda.synchronize()
    Cw, tol = oracle.gemm(oracle.dequantize_f64(fa, ca, sa, M, K), oracle.dequantize_f64(fb, cb, sb, N, K))
    return C.float().cpu().numpy(), Cw, tol


CASES = [(2, 2, True), (2, 2, False), (7, 7, False), (7, 2, False), (6, 2, False), (2, 7, False)]


@pytest.mark.parametrize("fa,fb,tiled", CASES)
@pytest.mark.parametrize("cdt", ["f32", "bf16"])
def test_nan_scale_codes(fa, fb, tiled, cdt):
    """Scale code 0xFF in a few blocks of A and B: NaN in exactly the rows
    and columns the oracle gives, the rest within the bound."""
    M, N, K = 320, 288 if not tiled else 512, 2048
    if tiled:
        M = 512
    g = np.random.default_rng(fa * 10 + fb + (100 if tiled else 0))
    ca, cb = _codes(g, fa, M, K), _codes(g, fb, N, K)
    sa = g.integers(118, 132, (M, K // 32)).astype(np.uint8)
    sb = g.integers(118, 132, (N, K // 32)).astype(np.uint8)
    for r, b in ((3, 0), (77, 5), (M - 1, K // 32 - 1)):
        sa[r, b] = 0xFF
    for r, b in ((0, 7), (N // 2, 11)):
        sb[r, b] = 0xFF
    got, Cw, tol = _run(fa, fb, ca, sa, cb, sb, M, N, K, tiled, cdt)
    assert np.isnan(Cw[3]).all() and np.isnan(Cw[:, 0]).all()
    check_gemm(got, Cw, tol, cdt == "bf16", f"NaN codes fa={fa} fb={fb} tiled={tiled} {cdt}")


def _grid_threshold(fa, fb):
    g = {1: 9, 5: 16, 7: 3, 6: 4, 2: 1}
    return 105 + g[fa] + g[fb]


@pytest.mark.parametrize("fa,fb,tiled", [(2, 2, True), (1, 1, True)])
@pytest.mark.parametrize("pattern", ["rows", "tile", "spread"])
def test_products_below_fp32_spacing(fa, fb, tiled, pattern):
    """Scale codes whose products fall below FP32's subnormal spacing:
    rows   -- some whole rows of A and B at low codes among ordinary rows;
    tile   -- every code of the first 256 x 256 output tile low;
    spread -- low rows next to high codes (products up to 2^56) in the same
              tiles.
    FP32 output, checked as the FP32 rounding of a value within the bound
    (MXFP8 pairs on the tile layout take the native FP8 instruction, whose
    documented bound is 1e-3 of sum |a b|)."""
    M, N, K = 512, 512, 2048
    g = np.random.default_rng({"rows": 1, "tile": 2, "spread": 3}[pattern] + 10 * fa)
    ca, cb = _codes(g, fa, M, K), _codes(g, fb, N, K)
    thr = _grid_threshold(fa, fb)
    sa = g.integers(110, 140, (M, K // 32)).astype(np.uint8)
    sb = g.integers(110, 140, (N, K // 32)).astype(np.uint8)
    if pattern == "rows":
        for r in (0, 5, 300):
            sa[r] = g.integers(20, 40, K // 32)
        for r in (1, 5, 400):
            sb[r] = g.integers(thr - 60, thr - 45, K // 32)
        sa[7] = 0  # all-zero-code row (2^-127 blocks) against ordinary B
    elif pattern == "tile":
        sa[:256] = g.integers(30, 45, (256, K // 32))
        sb[:256] = g.integers(30, 45, (256, K // 32))
    else:  # the raised pass must fit both ends into FP32's range
        hi = 150 if fa == 2 else 120  # FP8 products reach 2^18 more
        sa[:8] = g.integers(30, 40, (8, K // 32))
        sb[:8] = g.integers(40, 50, (8, K // 32))
        sa[100:104] = hi + g.integers(0, 10, (4, K // 32))
        sb[100:104] = hi - 10 + g.integers(0, 10, (4, K // 32))
    got, Cw, tol = _run(fa, fb, ca, sa, cb, sb, M, N, K, tiled, "f32")
    flags_tol = tol * (100.0 if fa in (1, 5) else 1.0)
    check_gemm(got, Cw, flags_tol, False, f"low codes fa={fa} fb={fb} {pattern}")
    low = {"rows": Cw[[0, 300]][:, [1, 400]], "tile": Cw[:256, :256], "spread": Cw[:8, :8]}[pattern]
    assert np.all(np.abs(low) < 2.0**-100)  # the planted products really are tiny


@pytest.mark.parametrize("fa,fb", [(2, 2)])
def test_products_at_the_fp32_spacing(fa, fb):
    """Every pair exactly at the threshold (products multiples of 2^-149):
    the first pass is already exact; one code lower needs the second pass."""
    M, N, K = 256, 256, 1024
    g = np.random.default_rng(9)
    ca, cb = _codes(g, fa, M, K), _codes(g, fb, N, K)
    thr = _grid_threshold(fa, fb)
    for s in (thr, thr - 1, thr - 20):
        sa = np.full((M, K // 32), s // 2, np.uint8)
        sb = np.full((N, K // 32), s - s // 2, np.uint8)
        got, Cw, tol = _run(fa, fb, ca, sa, cb, sb, M, N, K, True, "f32")
        check_gemm(got, Cw, tol, False, f"code sum {s}")


_LO = {1: 3, 5: 17, 4: 7, 6: 5}    # exact ranges of the 8-bit pipeline / E3M2 x E3M2 kernel
_HI = {1: 246, 5: 239, 4: 254, 6: 250}


def _range_case(fa, fb, K, below):
    M, N = (2048, 4096) if fa != 6 else (512, 512)  # sizes the 8-bit pipeline takes
    g = np.random.default_rng(fa * 100 + fb * 10 + K // 1024 + (7 if below else 0))
    ca, cb = _codes(g, fa, M, K), _codes(g, fb, N, K)
    # ordinary codes: A around 2^-25, B around 2^-65, so that one shift per
    # operand and tile fits every code of a tile into the exact range
    sa = g.integers(95 if fa == 5 else 100, 106 if fa == 5 else 111, (M, K // 32)).astype(np.uint8)
    sb = g.integers(55, 66, (N, K // 32)).astype(np.uint8)
    if below:
        sa[3] = _LO[fa] - 1
        sa[100] = 1
        sb[9] = _LO[fb] - 2
        sb[400] = max(1, _LO[fb] - 3)
    else:
        sa[300] = _HI[fa] + 1
    return _run(fa, fb, ca, sa, cb, sb, M, N, K, False, "f32")


@pytest.mark.parametrize("fa,fb", [(1, 1), (5, 1), (1, 5), (4, 4), (5, 5), (6, 6)])
@pytest.mark.parametrize("K", [1024, 2048])
def test_whole_rows_below_the_exact_code_range(fa, fb, K):
    """The exact 8-bit pipeline (E4M3 exact for scale codes 3..246, E5M2
    17..239, INT8 7..254) and E3M2 x E3M2 decoded to BF16 (5..250): whole rows
    of A and B at codes below those ranges, down to 1, among ordinary rows.
    The fix-up pass recomputes exactly those tiles, with each operand's codes
    shifted into the exact range and every product kept a normal FP32 value;
    FP32 out, checked in full."""
    got, Cw, tol = _range_case(fa, fb, K, True)
    check_gemm(got, Cw, tol, False, f"below fa={fa} fb={fb} K={K}")


@pytest.mark.parametrize("fa,fb", [(1, 1), (5, 1), (1, 5), (5, 5), (6, 6)])
def test_whole_row_above_the_exact_code_range(fa, fb):
    """One whole row of A one code above the range (INT8's ends at 254), its
    products kept finite by small B codes: recomputed with the codes shifted
    down."""
    got, Cw, tol = _range_case(fa, fb, 2048, False)
    check_gemm(got, Cw, tol, False, f"above fa={fa} fb={fb}")


@pytest.mark.parametrize("fa,fb", [(1, 1), (5, 1), (4, 4), (4, 1)])
def test_exact_8bit_pipeline_clean_operands_k4096(fa, fb):
    """Ordinary scale codes only, K = 4096 (a multiple of the fix-up scan's
    4096-word stride, and not): the fix-up pass recomputes nothing, so the
    pipelined kernel's own output is what is checked."""
    for M, N, K in ((1024, 768, 4096), (512, 512, 3072)):
        g = np.random.default_rng(fa * 10 + fb + K)
        ca, cb = _codes(g, fa, M, K), _codes(g, fb, N, K)
        sa = g.integers(118, 132, (M, K // 32)).astype(np.uint8)
        sb = g.integers(112, 126, (N, K // 32)).astype(np.uint8)
        got, Cw, tol = _run(fa, fb, ca, sa, cb, sb, M, N, K, False, "f32")
        check_gemm(got, Cw, tol, False, f"fa={fa} fb={fb} K={K}")


# Row-layout paths: the scaled instruction (MXFP4 on the pipelined and the
# simple kernel, FP6 pairs) and the kernels that decode to BF16 (E3M2 x E3M2,
# the exact 8-bit pipeline, the generic kernel for other pairs).
ROW_CASES = [
    (2, 2, 512, 512, 2048),     # MXFP4, simple kernel
    (2, 2, 320, 288, 1056),     # MXFP4, simple kernel, K/32 not a multiple of 16
    (2, 2, 2048, 4096, 1024),   # MXFP4, pipelined kernel
    (7, 7, 512, 512, 2048),     # FP6 pairs on the scaled instruction
    (7, 2, 512, 512, 2048),
    (6, 2, 512, 512, 2048),
    (2, 7, 512, 512, 1024),
    (6, 6, 512, 512, 2048),     # E3M2 x E3M2, decoded to BF16
    (1, 1, 320, 288, 1024),     # MXFP8, small-shape kernel
    (1, 1, 2048, 4096, 1024),   # exact 8-bit pipeline
    (5, 1, 2048, 4096, 1024),
    (4, 4, 2048, 4096, 1024),
    (1, 2, 320, 288, 1024),     # generic kernel (8-bit x FP4)
]


@pytest.mark.parametrize("fa,fb,M,N,K", ROW_CASES)
@pytest.mark.parametrize("pattern", ["rows", "tile"])
def test_row_layout_products_below_fp32_spacing(fa, fb, M, N, K, pattern):
    """Row layout, every exact path: scale codes inside each kernel's
    conversion range whose pairs put products below FP32's subnormal spacing
    (c_A + c_B < 105 + g_A + g_B), as whole rows among ordinary rows or as a
    whole 256 x 256 output tile.  FP32 out, checked in full as the FP32
    rounding of a value within the bound."""
    g = np.random.default_rng(fa * 1000 + fb * 100 + K // 32 + (5 if pattern == "tile" else 0))
    ca, cb = _codes(g, fa, M, K), _codes(g, fb, N, K)
    thr = _grid_threshold(fa, fb) if fa in (1, 5, 7, 6, 2) and fb in (1, 5, 7, 6, 2) else 117
    sa = g.integers(115, 135, (M, K // 32)).astype(np.uint8)
    sb = g.integers(115, 135, (N, K // 32)).astype(np.uint8)
    lo = 20 if fa not in (1, 4, 5, 6) else 25  # inside every kernel's conversion range
    if pattern == "rows":
        for r in (0, 5, M - 1):
            sa[r] = g.integers(lo, lo + 15, K // 32)
        for r in (1, 5, N - 2):
            sb[r] = g.integers(thr - lo - 30, thr - lo - 15, K // 32)
    else:
        sa[:256] = g.integers(thr // 2 - 30, thr // 2 - 15, (min(M, 256), K // 32))
        sb[:256] = g.integers(thr // 2 - 30, thr // 2 - 15, (min(N, 256), K // 32))
    got, Cw, tol = _run(fa, fb, ca, sa, cb, sb, M, N, K, False, "f32")
    check_gemm(got, Cw, tol, False, f"row layout low codes fa={fa} fb={fb} {M}x{N}x{K} {pattern}")
