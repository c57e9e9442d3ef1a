"""Seeded random cases against the oracle, a net under the targeted tests:

* quantizers: every format, both roundings, BF16 or FP32 input, row pitches
  wider than the row, Hadamard on or off, the ceil rule (MX), Four Over Six
  and 2-D blocks (NVFP4); Student-t values over ten decades with planted
  zeros.  Codes, scales and the NVFP4 tensor scale bit for bit;
* GEMMs: random shapes (ragged in M, N and K) for every class of operand
  pair, FP32 out, every entry checked within the bound; row-layout shapes
  past one 256 x 256 tile (the pipelined kernels); MXFP4 in the tile layout
  quantized on the GPU (codes and scales checked against the oracle), BF16 or
  FP32 out."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import check_gemm, dev, host, to_gpu_bf16, to_gpu_f32, upload
    from tests.tiles import untile_codes, untile_scales


def _quant_case(g, max_rows=200, max_blocks=40, tiled_share=0.0):
    tiled = tiled_share > 0 and g.random() < tiled_share  # no extra draw for the small cases
    fmt = int(g.choice([1, 2, 5])) if tiled else int(g.choice([1, 2, 3, 4, 5, 6, 7, 3, 3, 2]))
    blk = 16 if fmt == 3 else 32
    if tiled:  # the tile layout: rows % 32 == 0, cols % 1024 == 0
        rows, cols = 32 * int(g.integers(1, max_rows // 32 + 2)), 1024 * int(g.integers(1, 5))
    else:
        rows, cols = int(g.integers(1, max_rows)), blk * int(g.integers(1, max_blocks))
    bf16 = g.random() < 0.6
    pad = 0 if tiled else int(g.choice([0, 0, 8, 24]))
    rnd = int(g.integers(0, 2))
    rht = bool(g.random() < 0.4)
    variant, flags = 0, 0
    if fmt == 3:
        r = g.random()
        if r < 0.2 and rnd == 0:
            variant, flags = oracle.V_FOUR6, mx.MX_FLAG_FOUR_OVER_SIX
        elif r < 0.45:
            variant, flags = oracle.V_2D, mx.MX_FLAG_BLOCK_2D
    elif g.random() < 0.2:
        variant, flags = oracle.V_CEIL, mx.MX_FLAG_SCALE_CEIL
    if rht:
        flags |= mx.MX_FLAG_RHT16
    x = (g.standard_t(3, (rows, cols)) * 10.0 ** g.uniform(-6, 4)).astype(np.float32)
    if g.random() < 0.2:
        x[g.integers(0, rows, 3), g.integers(0, cols, 3)] = 0.0
    if bf16:
        xin = (x.view(np.uint32) >> 16).astype(np.uint16)  # BF16 by truncation
        xd = to_gpu_bf16(xin, pad)
    else:
        xin, xd = x, to_gpu_f32(x, pad)
    seed, counter, mask = int(g.integers(0, 2**40)), int(g.integers(0, 2**40)), int(g.integers(0, 65536))
    out = mx.empty(fmt, rows, cols, device=dev(), layout=mx.MX_LAYOUT_TILED if tiled else mx.MX_LAYOUT_ROWS)
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    mx.mx_quantize(xd, out, rnd, seed, counter, flags, mask, amax if fmt == 3 else None)
    torch.cuda.synchronize()
    c, s, ts = host(out)
    if tiled:
        c, s = untile_codes(c, rows, cols if fmt != 2 else cols // 2), untile_scales(s, rows, cols // 32)
    wc, ws, wts = oracle.quantize(xin, fmt, rnd, seed=seed, counter=counter, rht=rht, sign_mask=mask,
                                  variant=variant)
    ok = np.array_equal(c, wc) and np.array_equal(s, ws) and (fmt != 3 or float(ts[0]) == wts)
    return ok, dict(fmt=fmt, rows=rows, cols=cols, bf16=bf16, pad=pad, rnd=rnd, flags=flags)


@pytest.mark.parametrize("seed", [101, 202])
def test_random_quantize_cases(seed):
    g = np.random.default_rng(seed)
    bad = [case for ok, case in (_quant_case(g) for _ in range(300)) if not ok]
    assert not bad, f"{len(bad)} of 300 cases differ from the oracle, e.g. {bad[:3]}"


@pytest.mark.parametrize("seed", [111])
def test_random_quantize_cases_large(seed):
    """Larger shapes (grids of many workgroups, the grid-stride amax pass),
    row and tile layouts."""
    g = np.random.default_rng(seed)
    bad = [case for ok, case in (_quant_case(g, 1500, 300, 0.3) for _ in range(24)) if not ok]
    assert not bad, f"{len(bad)} of 24 cases differ from the oracle, e.g. {bad[:3]}"


PAIRS = [(1, 1), (2, 2), (3, 3), (5, 1), (4, 4), (7, 7), (6, 6), (7, 2), (1, 2), (6, 4)]


@pytest.mark.parametrize("seed", [303, 404])
def test_random_gemm_cases(seed):
    g = np.random.default_rng(seed)
    bad = []
    for _ in range(50):
        fa, fb = PAIRS[int(g.integers(0, len(PAIRS)))]
        M, N = int(g.integers(1, 300)), int(g.integers(1, 300))
        K = 32 * int(g.integers(1, 40))
        if (fa in (6, 7) or fb in (6, 7)) and g.random() < 0.5:
            K = 512 * int(g.integers(1, 3))
        A = W.normal_bf16(M, K, float(10.0 ** g.uniform(-3, 2)), int(g.integers(0, 1000)), 1)
        B = W.normal_bf16(N, K, float(10.0 ** g.uniform(-3, 2)), int(g.integers(0, 1000)), 2)
        qa, qb = oracle.quantize(A, fa), oracle.quantize(B, fb)
        ta, tb = upload(fa, qa[0], qa[1], qa[2]), upload(fb, qb[0], qb[1], qb[2])
        ta.cols = tb.cols = K
        C = torch.empty(M, N, dtype=torch.float32, device=dev())
        mx.mx_gemm(ta, tb, C)
        torch.cuda.synchronize()
        Ahat = oracle.dequantize_f64(fa, qa[0], qa[1], M, K) * (qa[2] if fa == 3 else 1.0)
        Bhat = oracle.dequantize_f64(fb, qb[0], qb[1], N, K) * (qb[2] if fb == 3 else 1.0)
        Cw, tol = oracle.gemm(Ahat, Bhat)
        try:
            check_gemm(C.cpu().numpy(), Cw, tol, False, f"{fa} x {fb} {M}x{N}x{K}")
        except AssertionError as e:
            bad.append(str(e)[:200])
    assert not bad, f"{len(bad)} of 50 products outside the bound: {bad[:2]}"


def _gemm_pair_case(g, fa, fb, M, N, K):
    A = W.normal_bf16(M, K, float(10.0 ** g.uniform(-3, 2)), int(g.integers(0, 1000)), 1)
    B = W.normal_bf16(N, K, float(10.0 ** g.uniform(-3, 2)), int(g.integers(0, 1000)), 2)
    qa, qb = oracle.quantize(A, fa), oracle.quantize(B, fb)
    ta, tb = upload(fa, qa[0], qa[1], qa[2]), upload(fb, qb[0], qb[1], qb[2])
    ta.cols = tb.cols = K
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm(ta, tb, C)
    torch.cuda.synchronize()
    Ahat = oracle.dequantize_f64(fa, qa[0], qa[1], M, K) * (qa[2] if fa == 3 else 1.0)
    Bhat = oracle.dequantize_f64(fb, qb[0], qb[1], N, K) * (qb[2] if fb == 3 else 1.0)
    Cw, tol = oracle.gemm(Ahat, Bhat)
    check_gemm(C.cpu().numpy(), Cw, tol, False, f"{fa} x {fb} {M}x{N}x{K}")


@pytest.mark.parametrize("seed", [505, 606])
def test_random_gemm_cases_past_one_tile(seed):
    g = np.random.default_rng(seed)
    pairs = PAIRS + [(5, 5), (1, 5)]
    bad = []
    for _ in range(16):
        fa, fb = pairs[int(g.integers(0, len(pairs)))]
        M, N = int(g.integers(257, 1100)), int(g.integers(257, 1100))
        K = 512 * int(g.integers(1, 5)) if g.random() < 0.7 else 32 * int(g.integers(1, 80))
        try:
            _gemm_pair_case(g, fa, fb, M, N, K)
        except AssertionError as e:
            bad.append(str(e)[:200])
    assert not bad, f"{len(bad)} of 16 products outside the bound: {bad[:2]}"


@pytest.mark.parametrize("seed", [707, 808])
def test_random_tiled_mxfp4_cases(seed):
    g = np.random.default_rng(seed)
    bad = []
    for _ in range(16):
        M, N = 32 * int(g.integers(1, 40)), 32 * int(g.integers(1, 40))
        K = 1024 * int(g.integers(1, 5))
        A = W.normal_bf16(M, K, float(10.0 ** g.uniform(-3, 2)), int(g.integers(0, 1000)), 1,
                          outlier_entries=0.002, outlier_mult=50.0)
        B = W.normal_bf16(N, K, float(10.0 ** g.uniform(-3, 2)), int(g.integers(0, 1000)), 2)
        qa = mx.empty(2, M, K, device=dev(), layout=mx.MX_LAYOUT_TILED)
        qb = mx.empty(2, N, K, device=dev(), layout=mx.MX_LAYOUT_TILED)
        mx.mx_quantize(to_gpu_bf16(A), qa)
        mx.mx_quantize(to_gpu_bf16(B), qb)
        cdt = torch.bfloat16 if g.random() < 0.5 else torch.float32
        C = torch.empty(M, N, dtype=cdt, device=dev())
        mx.mx_gemm(qa, qb, C)
        torch.cuda.synchronize()
        oa, ob = oracle.quantize(A, 2), oracle.quantize(B, 2)
        for q, o, R in ((qa, oa, M), (qb, ob, N)):
            c, sc, _ = host(q)
            if not (np.array_equal(untile_codes(c, R, K // 2), o[0]) and np.array_equal(untile_scales(sc, R, K // 32), o[1])):
                bad.append(f"tiled quantize {R}x{K}")
        Cw, tol = oracle.gemm(oracle.dequantize_f64(2, oa[0], oa[1], M, K), oracle.dequantize_f64(2, ob[0], ob[1], N, K))
        try:
            check_gemm(C.float().cpu().numpy(), Cw, tol, cdt == torch.bfloat16, f"tiled MXFP4 {M}x{N}x{K}")
        except AssertionError as e:
            bad.append(str(e)[:200])
    assert not bad, f"{len(bad)} of 16 tiled cases failed: {bad[:2]}"


@pytest.mark.parametrize("seed", [909])
def test_random_requant_cases(seed):
    """Requant-transpose on random shapes (rows % 32 == 0, cols % 16 == 0,
    ragged against the 128 x 64 tiles), both sources and both roundings,
    bit for bit."""
    g = np.random.default_rng(seed)
    bad = []
    for _ in range(24):
        rows, cols = 32 * int(g.integers(1, 30)), 16 * int(g.integers(1, 60))
        rnd = int(g.integers(0, 2))
        sd, ctr = int(g.integers(0, 1 << 40)), int(g.integers(0, 1 << 40))
        bits = W.normal_bf16(rows, cols, float(10.0 ** g.uniform(-3, 3)), int(g.integers(0, 1000)), 45,
                             outlier_entries=0.005, outlier_mult=30.0)
        out = mx.empty(1, cols, rows, device=dev())
        if g.random() < 0.5:
            nv = oracle.quantize(bits, 3, 0)
            mx.mx_requant_transpose(out, src=upload(3, nv[0], nv[1], nv[2]), rnd=rnd, seed=sd, counter=ctr)
            wc, ws = oracle.requant_transpose(rows, cols, rnd, seed=sd, counter=ctr, nvfp4=nv)
            what = "nvfp4"
        else:
            mx.mx_requant_transpose(out, x_bf16=to_gpu_bf16(bits, pad_cols=int(g.choice([0, 8, 24]))), rnd=rnd,
                                    seed=sd, counter=ctr)
            wc, ws = oracle.requant_transpose(rows, cols, rnd, seed=sd, counter=ctr, bf16=bits)
            what = "bf16"
        torch.cuda.synchronize()
        c, s, _ = host(out)
        if not (np.array_equal(s, ws) and np.array_equal(c, wc)):
            bad.append(f"{what} {rows}x{cols} rnd {rnd}")
    assert not bad, f"{len(bad)} of 24 requant cases differ from the oracle: {bad[:3]}"
