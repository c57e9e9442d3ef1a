"""GPU parity of the block-scaled GEMMs against the FP64 oracle on the
decoded operands: |C - C_oracle| <= 1e-5 * sum_k |a_k b_k| for FP32 output,
and C within [bf16(C_oracle - tol), bf16(C_oracle + tol)] for BF16 output."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import check_gemm, dev, upload


def _operands(fmt, M, N, K, seed, outliers=True):
    a = W.normal_bf16(M, K, 1.0, seed, 50, outlier_entries=0.002 if outliers else 0.0, outlier_mult=50)
    b = W.normal_bf16(N, K, 0.5, seed, 51)
    qa = oracle.quantize(a, fmt, 0)
    qb = oracle.quantize(b, fmt, 0)
    return qa, qb


def _oracle_gemm(fmt, qa, qb, M, N, K):
    Ad = oracle.dequantize_f64(fmt, qa[0], qa[1], M, K)
    Bd = oracle.dequantize_f64(fmt, qb[0], qb[1], N, K)
    post = 1.0
    if fmt == 3:
        post = float(np.float64(qa[2]) * np.float64(qb[2]))
    return oracle.gemm(Ad, Bd, post)


GEMM_SHAPES = [(32, 32, 32), (64, 96, 64), (130, 70, 96), (256, 256, 256), (257, 129, 544),
               (1, 300, 1024)]


@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("cdt", ["f32", "bf16"])
def test_gemm_within_tolerance(shape, fmt, cdt):
    M, N, K = shape
    qa, qb = _operands(fmt, M, N, K, M + N + K)
    A = upload(fmt, *qa)
    B = upload(fmt, *qb)
    C = torch.full((M, N + 3), float("nan"), dtype=torch.float32 if cdt == "f32" else torch.bfloat16,
                   device=dev())[:, :N]
    mx.mx_gemm(A, B, C)
    torch.cuda.synchronize()
    Chat, tol = _oracle_gemm(fmt, qa, qb, M, N, K)
    check_gemm(C.float().cpu().numpy(), Chat, tol, cdt == "bf16", f"fmt {fmt} {shape} {cdt}")


@pytest.mark.parametrize("gather", [False, True])
def test_grouped_nvfp4(gather):
    tokens, K, N, E, topk = 96, 256, 80, 5, 2
    X = W.normal_bf16(tokens, K, 1.0, 3, 52)
    row_index, offsets = W.uniform_topk_routing(tokens, E, topk, 3, 53)
    R = row_index.size
    Wb = [W.normal_bf16(N, K, 0.02, 3, 60 + e) for e in range(E)]
    qw = [oracle.quantize(w, 3, 0) for w in Wb]
    if gather:
        qx = oracle.quantize(X, 3, 0)
        A = upload(3, *qx)
        ri = torch.from_numpy(row_index).to(dev())
    else:
        Xr = X[row_index]
        qx = oracle.quantize(np.ascontiguousarray(Xr), 3, 0)
        A = upload(3, *qx)
        ri = None
    B = upload(3, np.concatenate([q[0] for q in qw]), np.concatenate([q[1] for q in qw]),
               np.array([q[2] for q in qw], np.float32))
    off = torch.from_numpy(offsets).to(dev())
    C = torch.empty(R, N, dtype=torch.bfloat16, device=dev())
    mx.mx_gemm_grouped(A, ri, R, B, E, off, C)
    torch.cuda.synchronize()
    Cg = C.float().cpu().numpy()
    Ad = oracle.dequantize_f64(3, qx[0], qx[1], qx[0].shape[0], K)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        rows = row_index[lo:hi] if gather else np.arange(lo, hi)
        Bd = oracle.dequantize_f64(3, qw[e][0], qw[e][1], N, K)
        Chat, tol = oracle.gemm(Ad[rows], Bd, float(np.float64(qx[2]) * np.float64(qw[e][2])))
        check_gemm(Cg[lo:hi], Chat, tol, True, f"expert {e}")


def test_grouped_nvfp4_empty_and_uneven_groups():
    K, N = 64, 32
    offsets = np.array([0, 0, 3, 3, 200, 201], np.int64)  # empty groups and a ragged one
    E = offsets.size - 1
    R = int(offsets[-1])
    X = W.normal_bf16(R, K, 1.0, 4, 54)
    qx = oracle.quantize(X, 3, 0)
    qw = [oracle.quantize(W.normal_bf16(N, K, 1.0, 4, 70 + e), 3, 0) for e in range(E)]
    A = upload(3, *qx)
    B = upload(3, np.concatenate([q[0] for q in qw]), np.concatenate([q[1] for q in qw]),
               np.array([q[2] for q in qw], np.float32))
    C = torch.empty(R, N, dtype=torch.float32, device=dev())
    mx.mx_gemm_grouped(A, None, R, B, E, torch.from_numpy(offsets).to(dev()), C)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy()
    Ad = oracle.dequantize_f64(3, qx[0], qx[1], R, K)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            Bd = oracle.dequantize_f64(3, qw[e][0], qw[e][1], N, K)
            Chat, tol = oracle.gemm(Ad[lo:hi], Bd, float(np.float64(qx[2]) * np.float64(qw[e][2])))
            check_gemm(Cg[lo:hi], Chat, tol, False, f"expert {e}")


def test_gemm_identity_closed_form():
    """A = identity in MXFP4 (1.0 coded with scale 2^0 after the 2^2 shift):
    C equals the decoded B transposed exactly."""
    K = 128
    eye = np.eye(K, dtype=np.float32)
    qa = oracle.quantize(eye, 2, 0)
    b = W.normal_bf16(64, K, 1.0, 5, 55)
    qb = oracle.quantize(b, 2, 0)
    C = torch.empty(K, 64, dtype=torch.float32, device=dev())
    mx.mx_gemm(upload(2, *qa), upload(2, *qb), C)
    torch.cuda.synchronize()
    Bd = oracle.dequantize_f64(2, qb[0], qb[1], 64, K)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), Bd.T)


@pytest.mark.parametrize("shape", [(64, 96, 64), (257, 129, 544), (512, 512, 2048)])
def test_mxfp8_native_fp8_path_within_hardware_bound(shape):
    """The opt-in native FP8 path: gfx950 sums each 8-product group in a
    window ~13 bits below the group's largest product (probed), so each group
    loses < 7 * 2^-13 of its own sum|ab|; the test bound is 1e-3 * sum|ab|."""
    M, N, K = shape
    qa, qb = _operands(1, M, N, K, M + 2 * N + K)
    C = torch.empty(M, N, dtype=torch.float32, device=dev())
    mx.mx_gemm_ex(upload(1, *qa), upload(1, *qb), C, mx.MX_GEMM_FP8_NATIVE)
    torch.cuda.synchronize()
    Chat, tol = _oracle_gemm(1, qa, qb, M, N, K)
    check_gemm(C.cpu().numpy(), Chat, tol * 100.0, False, f"native fp8 {shape}")


@pytest.mark.parametrize("fmt,flags,cdt", [(2, 0, "bf16"), (2, 0, "f32"), (1, 1, "bf16"), (1, 1, "f32"),
                                            (1, 0, "bf16"), (1, 0, "f32"), (3, 0, "bf16"), (3, 0, "f32")])
def test_pipelined_ragged_tiles_and_unaligned_ldc(fmt, flags, cdt):
    """Shapes large enough for the 256x256 pipelined kernels, with M and N not
    multiples of the tile and a C row pitch that is not 16-byte aligned (the
    epilogue then falls back to element stores).  MXFP8 runs the exact path
    (flags=0: FP8 stages converted to BF16 for the BF16 instruction) and the
    native FP8 path (flags=1), whose bound is 100x the exact one; NVFP4 its
    FP4 stages converted to FP16 with the E4M3 block scales applied."""
    M, N, K = 2900, 3000, 512
    qa, qb = _operands(fmt, M, N, K, 17)
    dt = torch.float32 if cdt == "f32" else torch.bfloat16
    C = torch.full((M, N + 3), float("nan"), dtype=dt, device=dev())[:, :N]
    mx.mx_gemm_ex(upload(fmt, *qa), upload(fmt, *qb), C, flags)
    torch.cuda.synchronize()
    Chat, tol = _oracle_gemm(fmt, qa, qb, M, N, K)
    check_gemm(C.float().cpu().numpy(), Chat, tol * (100.0 if flags else 1.0), cdt == "bf16",
               f"pipelined fmt {fmt} {cdt}")
    C2 = torch.full((M, N), float("nan"), dtype=dt, device=dev())
    mx.mx_gemm_ex(upload(fmt, *qa), upload(fmt, *qb), C2, flags)
    torch.cuda.synchronize()
    check_gemm(C2.float().cpu().numpy(), Chat, tol * (100.0 if flags else 1.0), cdt == "bf16",
               f"pipelined aligned fmt {fmt} {cdt}")


@pytest.mark.parametrize("cdt", ["bf16", "f32"])
def test_exact_mxfp8_special_scale_codes(cdt):
    """At a size that takes the pipelined exact MXFP8 kernel, E8M0 scale codes
    0 (2^-127, on nonzero codes) and 255 (NaN) in a few blocks of A and B:
    the tiles holding them are recomputed by the fix-up pass, so NaN reaches
    exactly the rows and columns the oracle gives, and everything else stays
    within the bound."""
    M, N, K = 2048, 4096, 512
    qa, qb = _operands(1, M, N, K, 29)
    sa, sb = qa[1].copy(), qb[1].copy()
    sa[5, 3] = 0
    sa[700, 10] = 255
    sb[1234, 7] = 0
    sb[3000, 2] = 255
    qa = (qa[0], sa)
    qb = (qb[0], sb)
    dt = torch.float32 if cdt == "f32" else torch.bfloat16
    C = torch.full((M, N), 7.0, dtype=dt, device=dev())
    mx.mx_gemm(upload(1, *qa), upload(1, *qb), C)
    torch.cuda.synchronize()
    Chat, tol = _oracle_gemm(1, qa, qb, M, N, K)
    got = C.float().cpu().numpy()
    nan_want = np.isnan(Chat)
    assert nan_want[700].all() and nan_want[:, 3000].all() and nan_want.sum() == N + M - 1
    assert np.isnan(got[nan_want]).all(), "NaN scale blocks must give NaN outputs"
    keep = ~nan_want
    assert not np.isnan(got[keep]).any()
    check_gemm(np.where(keep, got, 0.0), np.where(keep, Chat, 0.0), np.where(keep, tol, 1.0),
               cdt == "bf16", f"exact mxfp8 special scales {cdt}")


@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("cdt", ["bf16", "f32"])
def test_grouped_nvfp4_pipelined(gather, cdt):
    """Grouped NVFP4 at a size that takes the pipelined kernel (R x N >= 2^22,
    K a multiple of 256; K = 768 runs the loop once and both peeled steps),
    with an empty group and groups that do not fill their last row tile."""
    K, N = 768, 2048
    offsets = np.array([0, 700, 700, 1930, 2048], np.int64)
    E = offsets.size - 1
    R = int(offsets[-1])
    tokens = 1500
    X = W.normal_bf16(tokens, K, 1.0, 6, 56)
    rng = np.random.default_rng(6)
    row_index = rng.integers(0, tokens, R).astype(np.int32)
    qw = [oracle.quantize(W.normal_bf16(N, K, 0.05, 6, 80 + e), 3, 0) for e in range(E)]
    if gather:
        qx = oracle.quantize(X, 3, 0)
        ri = torch.from_numpy(row_index).to(dev())
    else:
        qx = oracle.quantize(np.ascontiguousarray(X[row_index]), 3, 0)
        ri = None
    A = upload(3, *qx)
    B = upload(3, np.concatenate([q[0] for q in qw]), np.concatenate([q[1] for q in qw]),
               np.array([q[2] for q in qw], np.float32))
    dt = torch.float32 if cdt == "f32" else torch.bfloat16
    C = torch.full((R, N), float("nan"), dtype=dt, device=dev())
    mx.mx_gemm_grouped(A, ri, R, B, E, torch.from_numpy(offsets).to(dev()), C)
    torch.cuda.synchronize()
    Cg = C.float().cpu().numpy()
    Ad = oracle.dequantize_f64(3, qx[0], qx[1], qx[0].shape[0], K)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = row_index[lo:hi] if gather else np.arange(lo, hi)
        Bd = oracle.dequantize_f64(3, qw[e][0], qw[e][1], N, K)
        Chat, tol = oracle.gemm(Ad[rows], Bd, float(np.float64(qx[2]) * np.float64(qw[e][2])))
        check_gemm(Cg[lo:hi], Chat, tol, cdt == "bf16", f"pipelined expert {e} gather={gather}")


@pytest.mark.parametrize("gather", [False, True])
def test_grouped_nvfp4_pipelined_short_last_tiles(gather):
    """Pipelined grouped NVFP4 whose groups end 10, 40, 150, 230 and 18 rows
    into their last row tile (rows past a group's end are clamped copies that
    are computed but never stored), with and without the row gather."""
    K, N = 512, 4096
    offsets = np.array([0, 266, 306, 968, 1198, 1216], np.int64)
    E = offsets.size - 1
    R = int(offsets[-1])
    tokens = 900
    X = W.normal_bf16(tokens, K, 1.0, 7, 57)
    rng = np.random.default_rng(7)
    row_index = rng.integers(0, tokens, R).astype(np.int32)
    qw = [oracle.quantize(W.normal_bf16(N, K, 0.05, 7, 90 + e), 3, 0) for e in range(E)]
    if gather:
        qx = oracle.quantize(X, 3, 0)
        ri = torch.from_numpy(row_index).to(dev())
    else:
        qx = oracle.quantize(np.ascontiguousarray(X[row_index]), 3, 0)
        ri = None
    A = upload(3, *qx)
    B = upload(3, np.concatenate([q[0] for q in qw]), np.concatenate([q[1] for q in qw]),
               np.array([q[2] for q in qw], np.float32))
    C = torch.full((R, N), float("nan"), dtype=torch.float32, device=dev())
    mx.mx_gemm_grouped(A, ri, R, B, E, torch.from_numpy(offsets).to(dev()), C)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy()
    Ad = oracle.dequantize_f64(3, qx[0], qx[1], qx[0].shape[0], K)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = row_index[lo:hi] if gather else np.arange(lo, hi)
        Bd = oracle.dequantize_f64(3, qw[e][0], qw[e][1], N, K)
        Chat, tol = oracle.gemm(Ad[rows], Bd, float(np.float64(qx[2]) * np.float64(qw[e][2])))
        check_gemm(Cg[lo:hi], Chat, tol, False, f"short-tile expert {e} gather={gather}")


# K = 0: every GEMM path writes the empty sum, C = 0, into exactly [M, N]
EMPTY_K_CASES = [  # (A format, B format, layout, flags)
    (2, 2, 0, 0), (2, 2, 1, 0), (1, 1, 0, 0), (1, 1, 0, 1), (1, 1, 1, 1), (3, 3, 0, 0),
    (5, 1, 0, 0), (5, 5, 1, 1), (4, 4, 0, 0), (7, 7, 0, 0), (6, 6, 0, 0), (7, 2, 0, 0)]


@pytest.mark.parametrize("fa,fb,layout,flags", EMPTY_K_CASES)
@pytest.mark.parametrize("cdt", [torch.float32, torch.bfloat16])
def test_empty_k_product_is_zero(fa, fb, layout, flags, cdt):
    M, N = 64, 96
    A = mx.empty(fa, M, 0, device=dev(), layout=layout)
    B = mx.empty(fb, N, 0, device=dev(), layout=layout)
    C = torch.full((M, N + 8), float("nan"), dtype=cdt, device=dev())
    mx.mx_gemm_ex(A, B, C[:, :N], flags)
    torch.cuda.synchronize()
    assert bool(torch.all(C[:, :N] == 0))
    assert bool(torch.all(torch.isnan(C[:, N:])))  # the pitch padding is not written


def test_empty_k_grouped_and_empty_rows():
    E, N = 4, 32
    A = mx.empty(3, 40, 0, device=dev())
    B = mx.empty(3, E * N, 0, device=dev(), n_tensor_scales=E)
    off = torch.tensor([0, 10, 10, 25, 40], dtype=torch.int64, device=dev())
    C = torch.full((40, N), float("nan"), dtype=torch.float32, device=dev())
    mx.mx_gemm_grouped(A, None, 40, B, E, off, C)
    torch.cuda.synchronize()
    assert bool(torch.all(C == 0))
    # no routed rows, or M = 0 on a plain GEMM: nothing is written
    C.fill_(float("nan"))
    mx.mx_gemm_grouped(mx.empty(3, 0, 64, device=dev()), None, 0, mx.empty(3, E * N, 64, device=dev(),
                       n_tensor_scales=E), E, torch.zeros(E + 1, dtype=torch.int64, device=dev()), C[:0])
    a0 = mx.empty(2, 0, 64, device=dev())
    mx.mx_gemm(a0, mx.empty(2, N, 64, device=dev()), C[:0])
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(C)))


@pytest.mark.parametrize("R,N,K,offsets", [
    (40, 32, 64, [0, 30, 20, 100]),                  # small shapes (staged kernel)
    (4096, 1024, 256, [0, 1000, 900, 5000, 6000]),   # the pipelined kernel
])
def test_grouped_offsets_outside_their_contract_stay_inside_c(R, N, K, offsets):
    """Group offsets that decrease or run past R (a broken caller) are
    clamped into [0, R] on the device: rows past C are never written."""
    E = len(offsets) - 1
    g = torch.Generator(device=dev()).manual_seed(3)
    x = torch.randn(R, K, device=dev(), generator=g).to(torch.bfloat16)
    w = torch.randn(E * N, K, device=dev(), generator=g).to(torch.bfloat16)
    A = mx.empty(3, R, K, device=dev())
    mx.mx_quantize(x, A, amax=torch.zeros(1, device=dev()))
    B = mx.empty(3, E * N, K, device=dev(), n_tensor_scales=E)
    for e in range(E):
        sub = mx.MXTensor(3, N, K, B.codes[e * N:(e + 1) * N], B.scales[e * N:(e + 1) * N],
                          B.tensor_scale[e:e + 1])
        mx.mx_quantize(w[e * N:(e + 1) * N], sub, amax=torch.zeros(1, device=dev()))
    big = torch.full((R + 64, N), float("nan"), dtype=torch.float32, device=dev())
    off = torch.tensor(offsets, dtype=torch.int64, device=dev())
    mx.mx_gemm_grouped(A, None, R, B, E, off, big[:R])
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(big[R:])))
    # rows that only the first group covers after the clamp match the same
    # call with offsets that keep the contract (same kernel, same tiles)
    ranges = []
    for e in range(E):
        lo = min(max(offsets[e], 0), R)
        ranges.append((lo, min(max(offsets[e + 1], lo), R)))
    cut = min([ranges[0][1]] + [lo for lo, hi in ranges[1:] if hi > lo])
    assert cut > 0
    good = torch.tensor([0, offsets[1]] + [R] * (E - 1), dtype=torch.int64, device=dev())
    ref = torch.empty(R, N, dtype=torch.float32, device=dev())
    mx.mx_gemm_grouped(A, None, R, B, E, good, ref)
    torch.cuda.synchronize()
    assert torch.equal(big[:cut], ref[:cut])
