"""Tensors past 32-bit offsets: a 66048 x 65536 BF16 tensor (8.7 GB, 4.3e9
elements) through the row-layout quantizers, the decode and both requant
kernels, so that input, code and output offsets all pass 2^32; and GEMMs
whose A operand holds 4.3 GB of codes (MXFP4 in both layouts, exact MXFP8,
grouped NVFP4 with a row gather).  Rows and
columns are sampled at both ends and compared with the oracle: codes bit for
bit (blocks are row-local, NVFP4 given the tensor's amax, requant bands
given the random counter where the band starts), products within the bound."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import check_gemm, dev

ROWS, COLS = 66048, 65536        # rows % 128 == 0: also a requant source
SAMPLE_ROWS = [0, 1, 32767, 65535, 65536, ROWS - 1]
BAND = 64                         # source columns per requant band


@pytest.fixture(scope="module")
def big():
    g = torch.Generator(device=dev()).manual_seed(11)
    x = torch.randn((ROWS, COLS), dtype=torch.bfloat16, device=dev(), generator=g)
    yield x
    del x
    torch.cuda.empty_cache()


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _host(t):
    return t.cpu().numpy()


def test_mxfp8_quantize_and_decode_past_32bit_offsets(big):
    q = mx.empty(mx.MX_MXFP8_E4M3, ROWS, COLS, device=dev())
    mx.mx_quantize(big, q)
    y = torch.empty_like(big)
    mx.mx_dequantize(q, y)
    torch.cuda.synchronize()
    rows = torch.tensor(SAMPLE_ROWS, device=dev())
    xs = _bits(big[rows])
    wc, ws, _ = oracle.quantize(xs, 1)
    assert np.array_equal(_host(q.codes[rows]), wc)
    assert np.array_equal(_host(q.scales[rows]), ws)
    ref = oracle.dequantize(1, wc, ws, None, len(SAMPLE_ROWS), COLS)
    assert np.array_equal(_bits(y[rows]), _bits(torch.from_numpy(ref).to(torch.bfloat16)))
    del q, y
    torch.cuda.empty_cache()


def test_nvfp4_amax_and_quantize_past_32bit_offsets(big):
    q = mx.empty(mx.MX_NVFP4, ROWS, COLS, device=dev())
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    mx.mx_quantize(big, q, amax=amax)
    torch.cuda.synchronize()
    T = float(amax.item())
    assert T == float(big.abs().max().float().item())
    rows = torch.tensor(SAMPLE_ROWS, device=dev())
    wc, ws, wts = oracle.quantize(_bits(big[rows]), 3, amax=T)
    assert float(q.tensor_scale.item()) == wts
    assert np.array_equal(_host(q.codes[rows]), wc)
    assert np.array_equal(_host(q.scales[rows]), ws)
    # requant of this NVFP4 source (SR): the last band of source columns
    out = mx.empty(mx.MX_MXFP8_E4M3, COLS, ROWS, device=dev())
    mx.mx_requant_transpose(out, src=q, rnd=mx.MX_SR, seed=5, counter=9)
    torch.cuda.synchronize()
    c0 = COLS - BAND
    band = (_host(q.codes[:, c0 // 2:]), _host(q.scales[:, c0 // 16:]), wts)
    oc, os_ = oracle.requant_transpose(ROWS, BAND, oracle.SR, 5, 9 + c0 * ROWS // 8, nvfp4=band)
    assert np.array_equal(_host(out.codes[c0:]), oc)
    assert np.array_equal(_host(out.scales[c0:]), os_)
    del q, out
    torch.cuda.empty_cache()


def test_bf16_requant_past_32bit_offsets(big):
    out = mx.empty(mx.MX_MXFP8_E4M3, COLS, ROWS, device=dev())
    mx.mx_requant_transpose(out, x_bf16=big, rnd=mx.MX_SR, seed=7, counter=3)
    torch.cuda.synchronize()
    for c0 in (0, COLS - BAND):
        xs = _bits(big[:, c0:c0 + BAND])
        oc, os_ = oracle.requant_transpose(ROWS, BAND, oracle.SR, 7, 3 + c0 * ROWS // 8, bf16=xs)
        assert np.array_equal(_host(out.codes[c0:c0 + BAND]), oc)
        assert np.array_equal(_host(out.scales[c0:c0 + BAND]), os_)
    del out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", [0, 1])
def test_mxfp4_gemm_operand_past_32bit_offsets(layout):
    """M = 66048, N = 512, K = 131072: A's codes span 4.3 GB.  Row layout:
    past the pipelined kernel's 32-bit offsets, so the general kernel and
    the fix-up scan run; tile layout: the register-direct kernel."""
    M, N, K = 66048, 512, 131072
    g = torch.Generator(device=dev()).manual_seed(12)
    a = torch.randn((M, K), dtype=torch.bfloat16, device=dev(), generator=g)
    b = torch.randn((N, K), dtype=torch.bfloat16, device=dev(), generator=g)
    qa = mx.empty(mx.MX_MXFP4_E2M1, M, K, device=dev(), layout=layout)
    qb = mx.empty(mx.MX_MXFP4_E2M1, N, K, device=dev(), layout=layout)
    mx.mx_quantize(a, qa)
    mx.mx_quantize(b, qb)
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm(qa, qb, C)
    torch.cuda.synchronize()
    rows, cols = [0, 32767, 65535, M - 1], [0, 1, 255, N - 1]
    ca, sa, _ = oracle.quantize(_bits(a[torch.tensor(rows, device=dev())]), 2)
    cb, sb, _ = oracle.quantize(_bits(b[torch.tensor(cols, device=dev())]), 2)
    Ad = oracle.dequantize_f64(2, ca, sa, len(rows), K)
    Bd = oracle.dequantize_f64(2, cb, sb, len(cols), K)
    ri = np.repeat(np.arange(len(rows)), len(cols))
    cj = np.tile(np.arange(len(cols)), len(rows))
    Chat, tol = oracle.gemm_sampled(Ad, Bd, ri, cj)
    got = C[torch.tensor(rows, device=dev())][:, torch.tensor(cols, device=dev())].cpu().numpy().reshape(-1)
    check_gemm(got, Chat, tol, False, f"layout {layout}")
    del a, b, qa, qb, C
    torch.cuda.empty_cache()


def test_exact_mxfp8_gemm_operand_past_32bit_offsets(big):
    """The 8.7 GB tensor as an MXFP8 A operand (4.3 GB of codes), N = 256:
    past the exact pipeline's 32-bit offsets, so the staged kernel and its
    fix-up pass run."""
    M, K, N = ROWS, COLS, 256
    qa = mx.empty(mx.MX_MXFP8_E4M3, M, K, device=dev())
    mx.mx_quantize(big, qa)
    g = torch.Generator(device=dev()).manual_seed(13)
    b = torch.randn((N, K), dtype=torch.bfloat16, device=dev(), generator=g)
    qb = mx.empty(mx.MX_MXFP8_E4M3, N, K, device=dev())
    mx.mx_quantize(b, qb)
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm(qa, qb, C)
    torch.cuda.synchronize()
    rows, cols = SAMPLE_ROWS, [0, 1, 128, N - 1]
    ca, sa, _ = oracle.quantize(_bits(big[torch.tensor(rows, device=dev())]), 1)
    cb, sb, _ = oracle.quantize(_bits(b[torch.tensor(cols, device=dev())]), 1)
    Ad = oracle.dequantize_f64(1, ca, sa, len(rows), K)
    Bd = oracle.dequantize_f64(1, cb, sb, len(cols), K)
    ri = np.repeat(np.arange(len(rows)), len(cols))
    cj = np.tile(np.arange(len(cols)), len(rows))
    Chat, tol = oracle.gemm_sampled(Ad, Bd, ri, cj)
    got = C[torch.tensor(rows, device=dev())][:, torch.tensor(cols, device=dev())].cpu().numpy().reshape(-1)
    check_gemm(got, Chat, tol, False, "exact MXFP8")
    del qa, qb, b, C
    torch.cuda.empty_cache()


def test_grouped_nvfp4_gather_past_32bit_offsets():
    """Grouped NVFP4 GEMM whose gathered A (66048 x 131072) holds 4.3 GB of
    codes; routed rows gather from both ends of A, two experts."""
    T, K, N, E = 66048, 131072, 256, 2
    g = torch.Generator(device=dev()).manual_seed(14)
    x = torch.randn((T, K), dtype=torch.bfloat16, device=dev(), generator=g)
    qx = mx.empty(mx.MX_NVFP4, T, K, device=dev())
    ax = torch.zeros(1, dtype=torch.float32, device=dev())
    mx.mx_quantize(x, qx, amax=ax)
    w = torch.randn((E * N, K), dtype=torch.bfloat16, device=dev(), generator=g)
    qw = mx.empty(mx.MX_NVFP4, E * N, K, device=dev(), n_tensor_scales=E)
    aw = torch.zeros(E, dtype=torch.float32, device=dev())
    for e in range(E):
        sub = mx.MXTensor(3, N, K, qw.codes[e * N:(e + 1) * N], qw.scales[e * N:(e + 1) * N],
                          qw.tensor_scale[e:e + 1])
        mx.mx_quantize(w[e * N:(e + 1) * N], sub, amax=aw[e:e + 1])
    R = 512
    src = np.concatenate([np.arange(T - 256, T), np.arange(256)]).astype(np.int32)  # far end first
    ri = torch.from_numpy(src).to(dev())
    off = torch.tensor([0, 256, R], dtype=torch.int64, device=dev())
    C = torch.empty(R, N, dtype=torch.float32, device=dev())
    mx.mx_gemm_grouped(qx, ri, R, qw, E, off, C)
    torch.cuda.synchronize()
    TA = float(ax.item())
    routed = [0, 255, 256, 511]
    cols = [0, 77, N - 1]
    xr = _bits(x[torch.from_numpy(src[routed].astype(np.int64)).to(dev())])
    cx, sx, ts_x = oracle.quantize(xr, 3, amax=TA)
    Ad = oracle.dequantize_f64(3, cx, sx, len(routed), K)
    for e in range(E):
        wr = _bits(w[torch.tensor([e * N + c for c in cols], device=dev())])
        cw, sw, ts_w = oracle.quantize(wr, 3, amax=float(aw[e].item()))
        Bd = oracle.dequantize_f64(3, cw, sw, len(cols), K)
        mine = [i for i, r in enumerate(routed) if (r >= 256) == (e == 1)]
        ri_ = np.repeat(np.array(mine), len(cols))
        cj_ = np.tile(np.arange(len(cols)), len(mine))
        Chat, tol = oracle.gemm_sampled(Ad, Bd, ri_, cj_, float(np.float64(ts_x) * np.float64(ts_w)))
        got = C[torch.tensor([routed[i] for i in mine], device=dev())][:, torch.tensor(cols, device=dev())]
        check_gemm(got.cpu().numpy().reshape(-1), Chat, tol, False, f"expert {e}")
    del x, qx, w, qw, C
    torch.cuda.empty_cache()
