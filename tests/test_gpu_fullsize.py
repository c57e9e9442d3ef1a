"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: quantizer codes and scales bit-exact over the whole tensors;
GEMM outputs checked against the FP64 oracle over the whole output where the
oracle's full product takes seconds (256^3, 4096^3), else on seeded samples
of entries it computes one by one (|C - C_oracle| <= 1e-5 * sum|ab|, outputs
inside the interval of their format's rounding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import check_gemm, dev, host, to_gpu_bf16, upload
    from tests.tiles import untile_codes, untile_scales


def _sample(M, N, n, seed):
    g = np.random.default_rng(seed)
    ri = g.integers(0, M, n)
    cj = g.integers(0, N, n)
    # always include the corners and tile edges
    ri[:4] = [0, M - 1, 0, M - 1]
    cj[:4] = [0, 0, N - 1, N - 1]
    return ri, cj


@pytest.fixture(scope="module")
def cfg2_data():
    A, B = W.cfg2(0, 4096)
    return A, B


@pytest.mark.parametrize("fmt", [2, 1])
def test_cfg2_quantize_bit_exact_full(cfg2_data, fmt):
    A, B = cfg2_data
    for x in (A, B):
        out = mx.empty(fmt, 4096, 4096, device=dev())
        mx.mx_quantize(to_gpu_bf16(x), out)
        torch.cuda.synchronize()
        c, s, _ = host(out)
        wc, ws, _ = oracle.quantize(x, fmt)
        assert np.array_equal(s, ws) and np.array_equal(c, wc)


def test_cfg1_quantize_gemm_end_to_end():
    """MXFP8 end to end at 256^3: A, B N(0,1) with 0.1% entries x100
    quantized on the GPU (E4M3, RNE; codes and scales bit-exact), then the
    block-scaled GEMM to FP32, every output entry against the oracle."""
    A, B = W.cfg1(0)
    M = N = K = 256
    qa = mx.empty(1, M, K, device=dev())
    qb = mx.empty(1, N, K, device=dev())
    mx.mx_quantize(to_gpu_bf16(A), qa)
    mx.mx_quantize(to_gpu_bf16(B), qb)
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm(qa, qb, C)
    torch.cuda.synchronize()
    oa, ob = oracle.quantize(A, 1), oracle.quantize(B, 1)
    for q, o in ((qa, oa), (qb, ob)):
        c, sc, _ = host(q)
        assert np.array_equal(sc, o[1]) and np.array_equal(c, o[0])
    Chat, tol = oracle.gemm(oracle.dequantize_f64(1, oa[0], oa[1], M, K),
                            oracle.dequantize_f64(1, ob[0], ob[1], N, K))
    check_gemm(C.cpu().numpy(), Chat, tol, False, "cfg1 256^3")


def test_cfg2_batch_quantize_and_tiled_gemm_full_output(cfg2_data):
    """The benchmark's step at full size: both cfg2 operands quantized to
    MXFP4 in the tile layout by one mx_quantize_batch call (codes and scales
    bit-exact against the oracle), then the tiled GEMM, BF16 out, every one
    of the 4096^2 outputs against the FP64 oracle."""
    A, B = cfg2_data
    M = N = K = 4096
    T = mx.MX_LAYOUT_TILED
    qa = mx.empty(2, M, K, device=dev(), layout=T)
    qb = mx.empty(2, N, K, device=dev(), layout=T)
    mx.mx_quantize_batch([dict(x=to_gpu_bf16(A), out=qa), dict(x=to_gpu_bf16(B), out=qb)])
    C = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    mx.mx_gemm(qa, qb, C)
    torch.cuda.synchronize()
    oa, ob = oracle.quantize(A, 2), oracle.quantize(B, 2)
    for q, o, R in ((qa, oa, M), (qb, ob, N)):
        c, sc, _ = host(q)
        assert np.array_equal(untile_scales(sc, R, K // 32), o[1])
        assert np.array_equal(untile_codes(c, R, K // 2), o[0])
    Chat, tol = oracle.gemm(oracle.dequantize_f64(2, oa[0], oa[1], M, K),
                            oracle.dequantize_f64(2, ob[0], ob[1], N, K))
    check_gemm(C.float().cpu().numpy(), Chat, tol, True, "tiled MXFP4 4096^3")


def test_cfg2_exact_mxfp8_gemm_full_output(cfg2_data):
    """MXFP8 (E4M3) 4096^3 on the exact path, BF16 out, every output entry
    against the FP64 oracle."""
    A, B = cfg2_data
    M = N = K = 4096
    qa, qb = oracle.quantize(A, 1), oracle.quantize(B, 1)
    C = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    mx.mx_gemm(upload(1, *qa), upload(1, *qb), C)
    torch.cuda.synchronize()
    Chat, tol = oracle.gemm(oracle.dequantize_f64(1, qa[0], qa[1], M, K),
                            oracle.dequantize_f64(1, qb[0], qb[1], N, K))
    check_gemm(C.float().cpu().numpy(), Chat, tol, True, "exact MXFP8 4096^3")


@pytest.mark.parametrize("fmt,flags,scale", [(2, 0, 1.0), (1, 0, 1.0), (1, 1, 100.0)])
def test_cfg2_gemm_4096_sampled(cfg2_data, fmt, flags, scale):
    """4096^3 GEMM in the benchmark's configuration (256x256 pipelined kernel),
    BF16 output; MXFP8 both exact and (flags=1) native FP8 with its 1e-3 bound."""
    A, B = cfg2_data
    M = N = K = 4096
    qa, qb = oracle.quantize(A, fmt), oracle.quantize(B, fmt)
    C = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    mx.mx_gemm_ex(upload(fmt, *qa), upload(fmt, *qb), C, flags)
    torch.cuda.synchronize()
    ri, cj = _sample(M, N, 4096, 7)
    Ad = oracle.dequantize_f64(fmt, qa[0], qa[1], M, K)
    Bd = oracle.dequantize_f64(fmt, qb[0], qb[1], N, K)
    Chat, tol = oracle.gemm_sampled(Ad, Bd, ri, cj)
    got = C.float().cpu().numpy()[ri, cj]
    check_gemm(got, Chat, tol * scale, True, f"fmt {fmt} flags {flags}")


@pytest.mark.parametrize("flags,scale", [(0, 1.0), (1, 100.0)])
def test_cfg4_wgrad_shape_sampled(flags, scale):
    """MXFP8 wgrad shape M=4096 N=14336 K=16384 with FP32 output on seeded
    N(0,1) operands quantized by the oracle: the exact path, and (flags=1)
    the native FP8 instruction with its 1e-3 bound."""
    M, N, K = 4096, 14336, 16384
    a = W.normal_bf16(M, K, 1.0, 1, 80)
    b = W.normal_bf16(N, K, 1.0, 1, 81)
    qa, qb = oracle.quantize(a, 1), oracle.quantize(b, 1)
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm_ex(upload(1, *qa), upload(1, *qb), C, flags)
    torch.cuda.synchronize()
    ri, cj = _sample(M, N, 2048, 8)
    Chat, tol = oracle.gemm_sampled(oracle.dequantize_f64(1, qa[0], qa[1], M, K),
                                    oracle.dequantize_f64(1, qb[0], qb[1], N, K), ri, cj)
    check_gemm(C.cpu().numpy()[ri, cj], Chat, tol * scale, False, f"wgrad flags {flags}")


def test_cfg3_grouped_full_sampled():
    """NVFP4 MoE forward at full size: 4096 tokens x 7168, top-8 of 32
    experts, W_e 2048 x 7168, row gather, BF16 out."""
    X, row_index, offsets, Ws = W.cfg3(0)
    E, N, K = 32, 2048, 7168
    R = int(offsets[-1])
    qx = oracle.quantize(X, 3)
    qw = [oracle.quantize(w, 3) for w in Ws]
    A = upload(3, *qx)
    B = upload(3, np.concatenate([q[0] for q in qw]), np.concatenate([q[1] for q in qw]),
               np.array([q[2] for q in qw], np.float32))
    C = torch.empty(R, N, dtype=torch.bfloat16, device=dev())
    mx.mx_gemm_grouped(A, torch.from_numpy(row_index).to(dev()), R, B, E,
                       torch.from_numpy(offsets).to(dev()), C)
    torch.cuda.synchronize()
    Cg = C.float().cpu().numpy()
    Ad = oracle.dequantize_f64(3, qx[0], qx[1], X.shape[0], K)
    g = np.random.default_rng(9)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = g.integers(lo, hi, 64)
        cols = g.integers(0, N, 64)
        Bd = oracle.dequantize_f64(3, qw[e][0], qw[e][1], N, K)
        Chat, tol = oracle.gemm_sampled(Ad, Bd, row_index[rows], cols,
                                        float(np.float64(qx[2]) * np.float64(qw[e][2])))
        check_gemm(Cg[rows, cols], Chat, tol, True, f"expert {e}")


def test_cfg5_rht_nvfp4_sr_full_bit_exact():
    G = W.cfg5(0)
    mask = mx.mx_rht_signs(0)
    out = mx.empty(3, G.shape[0], G.shape[1], device=dev())
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    mx.mx_quantize(to_gpu_bf16(G), out, mx.MX_SR, 0, 0, mx.MX_FLAG_RHT16, mask, amax)
    torch.cuda.synchronize()
    c, s, ts = host(out)
    wc, ws, wts = oracle.quantize(G, 3, oracle.SR, 0, 0, rht=True, sign_mask=mask)
    assert float(ts[0]) == wts
    assert np.array_equal(s, ws) and np.array_equal(c, wc)


def test_cfg4_requant_full_bit_exact():
    """Backward requant at full size, stochastic rounding: X (16384 x 4096,
    NVFP4) and dY (16384 x 14336, BF16) re-quantized transposed on the GPU in
    one launch each; every code and scale against the oracle.  dY's output
    is checked in bands of 2048 output rows (source columns), each band's
    oracle run starting its random counter where the band starts."""
    X, dY = W.cfg4(0, tokens=16384, hidden=4096, out=14336)
    nv = oracle.quantize(X, 3)
    out = mx.empty(1, 4096, 16384, device=dev())
    mx.mx_requant_transpose(out, src=upload(3, *nv), rnd=mx.MX_SR, seed=0, counter=0)
    torch.cuda.synchronize()
    c, s, _ = host(out)
    wc, ws = oracle.requant_transpose(16384, 4096, oracle.SR, 0, 0, nvfp4=nv)
    assert np.array_equal(s, ws) and np.array_equal(c, wc)
    del c, s, wc, ws, out
    rows, cols = dY.shape
    ctr = rows * 4096 // 8
    out2 = mx.empty(1, cols, rows, device=dev())
    mx.mx_requant_transpose(out2, x_bf16=to_gpu_bf16(dY), rnd=mx.MX_SR, seed=0, counter=ctr)
    torch.cuda.synchronize()
    c2, s2, _ = host(out2)
    band = 2048
    for c0 in range(0, cols, band):
        # output element n = oc * rows + orow draws counter + n / 8; a band
        # starting at output row c0 starts its oracle counter c0 * rows / 8 on
        wc2, ws2 = oracle.requant_transpose(rows, band, oracle.SR, 0, ctr + c0 * rows // 8,
                                            bf16=np.ascontiguousarray(dY[:, c0:c0 + band]))
        assert np.array_equal(s2[c0:c0 + band], ws2), f"scales, band {c0}"
        assert np.array_equal(c2[c0:c0 + band], wc2), f"codes, band {c0}"
