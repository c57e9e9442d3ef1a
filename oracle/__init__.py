"""CPU oracle for block-scaled quantization and block-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The product library never loads it and shares no code with it.

The arithmetic lives in ``mx_oracle.c`` (plain C, FP64 / exact FP32, encoders
that search the decoded alphabet).  This module compiles it with gcc and
wraps it with ctypes over numpy arrays.  Every function states which page
passage it follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MXFP8, MXFP4, NVFP4 = 1, 2, 3
# the other MX element types: INT8 (two's complement, 6 fraction bits; also the
# block-scaled "S2F6" combine format), FP8 E5M2, FP6 E3M2 and E2M3
MXINT8, MXFP8_E5M2, MXFP6_E3M2, MXFP6_E2M3 = 4, 5, 6, 7
RNE, SR = 0, 1
# quantizer variants (bits)
V_CEIL, V_FOUR6, V_2D = 1, 2, 4
IN_BF16, IN_F32 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile mx_oracle.c into liboracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _P(t):
    return ctypes.POINTER(t)


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    L = ctypes.CDLL(_LIB)
    c_u8p, c_f32p, c_f64p = _P(ctypes.c_uint8), _P(ctypes.c_float), _P(ctypes.c_double)
    i64, u64, u32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32
    vp, ci = ctypes.c_void_p, ctypes.c_int
    sig = {
        "mxo_init": (ci, []),
        "mxo_e2m1_decode": (ctypes.c_double, [u32]),
        "mxo_e4m3_decode": (ctypes.c_double, [u32]),
        "mxo_e8m0_decode": (ctypes.c_double, [u32]),
        "mxo_e5m2_decode": (ctypes.c_double, [u32]),
        "mxo_e3m2_decode": (ctypes.c_double, [u32]),
        "mxo_e2m3_decode": (ctypes.c_double, [u32]),
        "mxo_int8_decode": (ctypes.c_double, [u32]),
        "mxo_elem_decode": (ctypes.c_double, [ci, u32]),
        "mxo_elem_encode_rne": (u32, [ci, ctypes.c_double]),
        "mxo_elem_encode_sr": (u32, [ci, ctypes.c_double, u32]),
        "mxo_e2m1_encode_rne": (u32, [ctypes.c_double]),
        "mxo_e4m3_encode_rne": (u32, [ctypes.c_double]),
        "mxo_e2m1_encode_sr": (u32, [ctypes.c_double, u32]),
        "mxo_e4m3_encode_sr": (u32, [ctypes.c_double, u32]),
        "mxo_philox4x32_10": (None, [_P(ctypes.c_uint32), _P(ctypes.c_uint32), _P(ctypes.c_uint32)]),
        "mxo_rand16": (u32, [u64, u64, u64]),
        "mxo_rht_signs": (u32, [u64]),
        "mxo_rht16": (None, [vp, ci, c_f32p, i64, i64, u32, ci]),
        "mxo_quantize_mx": (ci, [vp, ci, i64, i64, i64, ci, ci, u64, u64, ci, u32, ci, c_u8p, c_u8p]),
        "mxo_tensor_amax": (ctypes.c_float, [vp, ci, i64, i64, i64, ci, u32]),
        "mxo_quantize_nvfp4": (ci, [vp, ci, i64, i64, i64, ci, u64, u64, ci, u32, ci, c_f32p,
                                    c_u8p, c_u8p, c_f32p]),
        "mxo_dequantize": (None, [ci, c_u8p, c_u8p, c_f32p, i64, i64, c_f32p]),
        "mxo_dequantize_f64": (None, [ci, c_u8p, c_u8p, i64, i64, c_f64p]),
        "mxo_requant_transpose": (ci, [ci, vp, c_u8p, c_f32p, i64, i64, ci, u64, u64, c_u8p, c_u8p]),
        "mxo_gemm_f64": (None, [c_f64p, c_f64p, i64, i64, i64, ctypes.c_double, c_f64p, c_f64p]),
        "mxo_gemm_f64_sampled": (None, [c_f64p, c_f64p, i64, _P(i64), _P(i64), i64,
                                        ctypes.c_double, c_f64p, c_f64p]),
        "mxo_encode_elems": (None, [ci, ci, c_f64p, _P(u64), i64, u64, u64, c_u8p]),
        "mxo_codes_bytes": (i64, [ci, i64, i64]),
        "mxo_scales_bytes": (i64, [ci, i64, i64]),
        "mxo_tensor_bytes": (i64, [ci, i64, i64]),
        "mxo_nv_sq_error_cmp": (ci, [c_f32p, c_u8p, u32, c_u8p, u32, ctypes.c_float]),
        "mxo_set_threads": (None, [ci]),
        "mxo_get_threads": (ci, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    L.mxo_init()
    _lib = L
    return L


def _ptr(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_P(t))


def _vptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _in(x: np.ndarray):
    """Input matrix as (array, dtype code).  bf16 data is passed as uint16 bits."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), IN_BF16
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), IN_F32
    raise TypeError("oracle inputs are bf16 bits (uint16) or float32")


# --- scalar codecs ---------------------------------------------------------
def e2m1_decode(code: int) -> float:
    return lib().mxo_e2m1_decode(code)


def e4m3_decode(code: int) -> float:
    return lib().mxo_e4m3_decode(code)


def e8m0_decode(code: int) -> float:
    return lib().mxo_e8m0_decode(code)


def e2m1_encode_rne(y: float) -> int:
    return lib().mxo_e2m1_encode_rne(y)


def e4m3_encode_rne(y: float) -> int:
    return lib().mxo_e4m3_encode_rne(y)


def e2m1_encode_sr(y: float, r16: int) -> int:
    return lib().mxo_e2m1_encode_sr(y, r16)


def e4m3_encode_sr(y: float, r16: int) -> int:
    return lib().mxo_e4m3_encode_sr(y, r16)


def elem_decode(fmt: int, code: int) -> float:
    """Value of one element code of MX format fmt (any MX format above)."""
    return lib().mxo_elem_decode(fmt, code)


def elem_encode_rne(fmt: int, y: float) -> int:
    return lib().mxo_elem_encode_rne(fmt, y)


def elem_encode_sr(fmt: int, y: float, r16: int) -> int:
    return lib().mxo_elem_encode_sr(fmt, y, r16)


def philox4x32_10(ctr, key):
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib().mxo_philox4x32_10(c, k, o)
    return [o[i] for i in range(4)]


def rand16(seed: int, counter: int, n: int) -> int:
    return lib().mxo_rand16(seed, counter, n)


def encode_elems(fmt: int, y: np.ndarray, rnd: int = RNE, n=None, seed: int = 0,
                 counter: int = 0) -> np.ndarray:
    """Element codes (the element type of MX format fmt) of the float64 values y,
    by RNE or by SR with the random value of element index n[t]."""
    y = np.ascontiguousarray(y, np.float64).ravel()
    idx = np.zeros(y.size, np.uint64) if n is None else np.ascontiguousarray(n, np.uint64).ravel()
    out = np.zeros(y.size, np.uint8)
    lib().mxo_encode_elems(fmt, rnd, _ptr(y, ctypes.c_double), _ptr(idx, ctypes.c_uint64), y.size,
                           seed, counter, _ptr(out, ctypes.c_uint8))
    return out


def rht_signs(seed: int) -> int:
    return lib().mxo_rht_signs(seed)


# --- tensor operations -----------------------------------------------------
def rht16(x: np.ndarray, sign_mask: int, inverse: bool = False) -> np.ndarray:
    x, dt = _in(x)
    rows, cols = x.shape
    assert cols % 16 == 0
    y = np.empty((rows, cols), np.float32)
    lib().mxo_rht16(_vptr(x), dt, _ptr(y, ctypes.c_float), rows, cols, sign_mask, int(inverse))
    return y


def codes_bytes(fmt, rows, cols):
    return lib().mxo_codes_bytes(fmt, rows, cols)


def scales_bytes(fmt, rows, cols):
    return lib().mxo_scales_bytes(fmt, rows, cols)


def tensor_bytes(fmt, rows, cols):
    return lib().mxo_tensor_bytes(fmt, rows, cols)


def tensor_amax(x: np.ndarray, rht: bool = False, sign_mask: int = 0) -> float:
    x, dt = _in(x)
    rows, cols = x.shape
    return float(lib().mxo_tensor_amax(_vptr(x), dt, cols, rows, cols, int(rht), sign_mask))


def quantize(x: np.ndarray, fmt: int, rnd: int = RNE, seed: int = 0, counter: int = 0,
             rht: bool = False, sign_mask: int = 0, amax: float | None = None,
             variant: int = 0):
    """Quantize a [rows, cols] matrix along cols.

    ``variant`` is a set of V_* bits: V_CEIL (MX formats: the smallest shared
    scale that saturates no element), V_FOUR6 (NVFP4, round-to-nearest: each
    block's maximum mapped to 4 or 6, whichever decodes with less error),
    V_2D (NVFP4: one block scale per 16 x 16 tile).

    Returns (codes, scales, tensor_scale): codes uint8 [rows, cols] (MXFP8) or
    [rows, cols/2] (FP4, element 2j in the low nibble); scales uint8
    [rows, cols/32] (E8M0) or [rows, cols/16] (E4M3); tensor_scale a float
    (NVFP4) or None.
    """
    x, dt = _in(x)
    rows, cols = x.shape
    cb = codes_bytes(fmt, rows, cols) // max(rows, 1)
    codes = np.zeros((rows, cb), np.uint8)
    if fmt == NVFP4:
        scales = np.zeros((rows, cols // 16), np.uint8)
        ts = np.zeros(1, np.float32)
        am = None if amax is None else np.array([amax], np.float32)
        rc = lib().mxo_quantize_nvfp4(_vptr(x), dt, cols, rows, cols, rnd, seed, counter, int(rht),
                                      sign_mask, variant,
                                      None if am is None else _ptr(am, ctypes.c_float),
                                      _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                                      _ptr(ts, ctypes.c_float))
        if rc:
            raise ValueError("oracle rejected the shape")
        return codes, scales, float(ts[0])
    scales = np.zeros((rows, cols // 32), np.uint8)
    rc = lib().mxo_quantize_mx(_vptr(x), dt, cols, rows, cols, fmt, rnd, seed, counter, int(rht),
                               sign_mask, variant, _ptr(codes, ctypes.c_uint8),
                               _ptr(scales, ctypes.c_uint8))
    if rc:
        raise ValueError("oracle rejected the shape")
    return codes, scales, None


def set_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops."""
    lib().mxo_set_threads(int(n))


def get_threads() -> int:
    return int(lib().mxo_get_threads())


def nv_sq_error_cmp(v: np.ndarray, codes_a, sb_a: int, codes_b, sb_b: int, S: float) -> int:
    """Sign of (exact squared error of encoding a) - (that of encoding b) for
    one 16-element NVFP4 block: v float32[16], codes 16 E2M1 codes each, sb
    the E4M3 block-scale codes, S the tensor scale."""
    v = np.ascontiguousarray(v, np.float32)
    ca = np.ascontiguousarray(codes_a, np.uint8)
    cb = np.ascontiguousarray(codes_b, np.uint8)
    assert v.shape == ca.shape == cb.shape == (16,)
    return int(lib().mxo_nv_sq_error_cmp(_ptr(v, ctypes.c_float), _ptr(ca, ctypes.c_uint8), sb_a,
                                         _ptr(cb, ctypes.c_uint8), sb_b, S))


def dequantize(fmt: int, codes: np.ndarray, scales: np.ndarray, tensor_scale, rows: int,
               cols: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    ts = np.array([tensor_scale if tensor_scale is not None else 1.0], np.float32)
    y = np.empty((rows, cols), np.float32)
    lib().mxo_dequantize(fmt, _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                         _ptr(ts, ctypes.c_float), rows, cols, _ptr(y, ctypes.c_float))
    return y


def dequantize_f64(fmt: int, codes: np.ndarray, scales: np.ndarray, rows: int,
                   cols: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    y = np.empty((rows, cols), np.float64)
    lib().mxo_dequantize_f64(fmt, _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                             rows, cols, _ptr(y, ctypes.c_double))
    return y


def requant_transpose(rows: int, cols: int, rnd: int = SR, seed: int = 0, counter: int = 0,
                      nvfp4=None, bf16: np.ndarray | None = None):
    """Source [rows, cols] (an NVFP4 (codes, scales, S) triple, or bf16 bits)
    -> MXFP8 codes [cols, rows] and E8M0 scales [cols, rows/32]."""
    codes = np.zeros((cols, rows), np.uint8)
    scales = np.zeros((cols, rows // 32), np.uint8)
    if nvfp4 is not None:
        c, s, ts = nvfp4
        c = np.ascontiguousarray(c, np.uint8)
        s = np.ascontiguousarray(s, np.uint8)
        tsa = np.array([ts], np.float32)
        rc = lib().mxo_requant_transpose(NVFP4, _vptr(c), _ptr(s, ctypes.c_uint8),
                                         _ptr(tsa, ctypes.c_float), rows, cols, rnd, seed, counter,
                                         _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8))
    else:
        b = np.ascontiguousarray(bf16, np.uint16)
        rc = lib().mxo_requant_transpose(0, _vptr(b), None, None, rows, cols, rnd, seed, counter,
                                         _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8))
    if rc:
        raise ValueError("oracle rejected the shape")
    return codes, scales


def gemm(A: np.ndarray, B: np.ndarray, post_scale: float = 1.0):
    """FP64 C = A @ B.T over decoded operands, and tol = 1e-5 * sum|a*b|."""
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    M, K = A.shape
    N = B.shape[0]
    C = np.empty((M, N), np.float64)
    T = np.empty((M, N), np.float64)
    lib().mxo_gemm_f64(_ptr(A, ctypes.c_double), _ptr(B, ctypes.c_double), M, N, K,
                       float(post_scale), _ptr(C, ctypes.c_double), _ptr(T, ctypes.c_double))
    return C, T


def gemm_sampled(A: np.ndarray, B: np.ndarray, ri: np.ndarray, cj: np.ndarray,
                 post_scale: float = 1.0):
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    ri = np.ascontiguousarray(ri, np.int64)
    cj = np.ascontiguousarray(cj, np.int64)
    n = ri.size
    C = np.empty(n, np.float64)
    T = np.empty(n, np.float64)
    lib().mxo_gemm_f64_sampled(_ptr(A, ctypes.c_double), _ptr(B, ctypes.c_double), A.shape[1],
                               _ptr(ri, ctypes.c_int64), _ptr(cj, ctypes.c_int64), n,
                               float(post_scale), _ptr(C, ctypes.c_double), _ptr(T, ctypes.c_double))
    return C, T


def bf16_interval(C: np.ndarray, tol: np.ndarray):
    """BF16-output acceptance interval [bf16_rne(C - tol), bf16_rne(C + tol)]
    as float64 arrays (the rounding here is the plain definition: nearest
    bf16, ties to even, computed through float32 which is exact for the
    bounds' own rounding because it is done on the FP64 value directly)."""
    lo = _round_bf16_f64(C - tol)
    hi = _round_bf16_f64(C + tol)
    return lo, hi


def roundtrip_stats(x: np.ndarray, y: np.ndarray):
    """Round-trip error statistics of a decoded tensor y against its source x
    ("Microscaling (MX) and block-scaled 4-bit formats", section "NVFP4" and
    glossary "stochastic rounding": what the Hadamard transform and stochastic
    rounding buy).  x: bf16 bits (uint16) or float32; y: float32 or float64,
    same shape.  Returns (sum (y-x)^2, sum x^2, sum (y-x), max |y-x|), every
    term formed and summed in FP64."""
    xv = bf16_bits_to_f64(x) if x.dtype == np.uint16 else np.asarray(x, np.float64)
    d = np.asarray(y, np.float64) - xv
    return float(np.sum(d * d)), float(np.sum(xv * xv)), float(np.sum(d)), float(np.max(np.abs(d)))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_interval(C: np.ndarray, tol: np.ndarray):
    """FP32-output acceptance interval [fp32_rne(C - tol), fp32_rne(C + tol)]
    as float64 arrays: the FP32 values that are the rounding of some value
    within the bound.  Where C +- tol are FP32 values this is the bound
    itself; it differs only where the bound is narrower than FP32's spacing
    (results in or below FP32's subnormal range)."""
    C = np.asarray(C, np.float64)
    tol = np.asarray(tol, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        lo = (C - tol).astype(np.float32).astype(np.float64)
        hi = (C + tol).astype(np.float32).astype(np.float64)
    return lo, hi


def _round_bf16_f64(v: np.ndarray) -> np.ndarray:
    """Round FP64 values to the nearest bf16 (ties to even), returned as FP64.

    Done in exact integer arithmetic on the FP64 significand so no double
    rounding through FP32 occurs."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)  # v = m * 2^e, |m| in [0.5, 1)
    # bf16 keeps 8 significant bits: scale to an integer significand of 8 bits
    # for normal values; clamp the exponent at the bf16 normal minimum (2^-126)
    # so subnormals keep fewer bits.
    e_min = -125  # smallest e (frexp convention) of a normal bf16
    bits = 8 - np.maximum(e_min - e, 0)
    bits = np.maximum(bits, 0)
    scaled = np.ldexp(m, bits)  # exact
    r = np.rint(scaled)  # round half to even (numpy rint)
    out = np.ldexp(r, e - bits)
    # overflow to inf beyond the bf16 max
    big = np.abs(out) > 3.3895313892515355e38
    out = np.where(big, np.sign(out) * np.inf, out)
    return out
