"""The C-ABI library loads without a GPU, exports every function that
include/mx.h declares, and rejects bad arguments on the host (no device work
happens for a rejected call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mx():
    import microscaling_precision_gemm_amd as mx
    if not os.path.exists(mx.LIB_PATH):
        from microscaling_precision_gemm_amd.build import build
        build()
    mx.load()
    return mx


def header_functions():
    src = open(os.path.join(ROOT, "include", "mx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_header_declares_the_binding_list(mx):
    assert header_functions() == sorted(mx.EXPORTED)


def test_library_exports_every_declared_symbol(mx):
    L = mx.load()
    for name in header_functions():
        assert hasattr(L, name), name


def test_host_helpers(mx, orc):
    for fmt, rows, cols in ((1, 3, 64), (2, 5, 96), (3, 7, 48)):
        assert mx.mx_codes_bytes(fmt, rows, cols) == orc.codes_bytes(fmt, rows, cols)
        assert mx.mx_scales_bytes(fmt, rows, cols) == orc.scales_bytes(fmt, rows, cols)
    assert mx.mx_codes_bytes(9, 4, 32) == 0
    for seed in (0, 1, 2**40 + 5):
        assert mx.mx_rht_signs(seed) == orc.rht_signs(seed)
    assert mx.load().mx_status_string(2) == b"inconsistent or unsupported shape"


FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails its checks


def _t(mx, fmt, rows, cols, codes=FAKE, scales=FAKE, ts=FAKE):
    return mx._Tensor(fmt, 0, rows, cols, codes, scales, ts)


def test_quantize_argument_checks(mx):
    L = mx.load()
    rng = mx._Rng(0, 0)
    t = _t(mx, 1, 4, 64)
    q = lambda *a: L.mx_quantize(*a)
    assert q(FAKE, 0, 4, 64, 64, None, 0, rng, 0, 0, None, None) == 1            # out NULL
    assert q(None, 0, 4, 64, 64, ctypes.byref(t), 0, rng, 0, 0, None, None) == 1  # x NULL
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(t), 7, rng, 0, 0, None, None) == 4  # rounding
    assert q(FAKE, 5, 4, 64, 64, ctypes.byref(t), 0, rng, 0, 0, None, None) == 4  # dtype
    assert q(FAKE, 0, 4, 64, 32, ctypes.byref(t), 0, rng, 0, 0, None, None) == 2  # ld < cols
    assert q(FAKE + 4, 0, 4, 64, 64, ctypes.byref(t), 0, rng, 0, 0, None, None) == 3  # align
    assert q(FAKE, 0, 4, 64, 68, ctypes.byref(t), 0, rng, 0, 0, None, None) == 3  # row pitch
    bad = _t(mx, 1, 4, 48)
    assert q(FAKE, 0, 4, 48, 48, ctypes.byref(bad), 0, rng, 0, 0, None, None) == 2  # 48 % 32
    wrong = _t(mx, 1, 5, 64)
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(wrong), 0, rng, 0, 0, None, None) == 2  # rows
    fmt = _t(mx, 9, 4, 64)
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(fmt), 0, rng, 0, 0, None, None) == 4
    nv = _t(mx, 3, 4, 64)
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(nv), 0, rng, 0, 0, None, None) == 1  # amax NULL
    nots = _t(mx, 3, 4, 64, ts=None)
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(nots), 0, rng, 0, 0, FAKE, None) == 1
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(t), 0, rng, 64, 0, None, None) == 5  # flags
    # variants: ceil is MX-only; Four Over Six is NVFP4 + RNE, not with 2-D; 2-D is NVFP4-only
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(nv), 0, rng, 4, 0, FAKE, None) == 5
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(t), 0, rng, 8, 0, None, None) == 5
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(t), 0, rng, 16, 0, None, None) == 5
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(nv), 1, rng, 8, 0, FAKE, None) == 5
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(nv), 0, rng, 8 | 16, 0, FAKE, None) == 5
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(t), 0, rng, 2, 0, None, None) == 5  # amax on MX
    nocodes = _t(mx, 1, 4, 64, codes=None)
    assert q(FAKE, 0, 4, 64, 64, ctypes.byref(nocodes), 0, rng, 0, 0, None, None) == 1


def test_quantize_batch_checks(mx):
    """Every job is checked before anything is enqueued: a bad job after a
    good one returns the bad job's status (without a GPU an enqueued launch
    would have returned MX_ERR_HIP instead)."""
    L = mx.load()
    assert L.mx_quantize_batch(None, 0, None) == 0
    assert L.mx_quantize_batch(None, 2, None) == 1
    assert L.mx_quantize_batch(None, -1, None) == 2
    good = mx._Tensor(2, 1, 32, 1024, FAKE, FAKE, None)
    bad = _t(mx, 1, 4, 48)
    jobs = (mx._Job * 2)()
    jobs[0] = mx._Job(FAKE, 0, 32, 1024, 1024, ctypes.pointer(good), 0, mx._Rng(0, 0), 0, 0, None)
    jobs[1] = mx._Job(FAKE, 0, 4, 48, 48, ctypes.pointer(bad), 0, mx._Rng(0, 0), 0, 0, None)
    assert L.mx_quantize_batch(jobs, 2, None) == 2
    jobs[1] = mx._Job(FAKE, 0, 32, 1024, 1024, ctypes.pointer(good), 0, mx._Rng(0, 0), 64, 0, None)
    assert L.mx_quantize_batch(jobs, 2, None) == 5


def test_quantize_batch_noalloc_checks(mx):
    """The no-allocation batch rejects, before any HIP call, more jobs than
    its slot array holds, a caller's amax buffer and MX_FLAG_AMAX_GIVEN."""
    L = mx.load()
    f = L.mx_quantize_batch_noalloc
    assert f(None, 0, None) == 0
    assert f(None, 2, None) == 1
    assert f(None, -1, None) == 2
    assert f(None, mx.MX_NOALLOC_MAX_JOBS + 1, None) == 2
    nv = mx._Tensor(3, 0, 4, 64, FAKE, FAKE, FAKE)
    jobs = (mx._Job * 2)()
    jobs[0] = mx._Job(FAKE, 0, 4, 64, 64, ctypes.pointer(nv), 0, mx._Rng(0, 0), 0, 0, None)
    jobs[1] = mx._Job(FAKE, 0, 4, 64, 64, ctypes.pointer(nv), 0, mx._Rng(0, 0), 0, 0, FAKE)
    assert f(jobs, 2, None) == 5  # a job brings its own amax slot
    jobs[1] = mx._Job(FAKE, 0, 4, 64, 64, ctypes.pointer(nv), 0, mx._Rng(0, 0), 2, 0, None)
    assert f(jobs, 2, None) == 5  # MX_FLAG_AMAX_GIVEN: there is no caller amax to read


def test_gemm_format_pair_checks(mx):
    """Mixed formats and the other MX element types: row layout, no flags, no
    NVFP4 in the pair."""
    L = mx.load()
    g = lambda A, B, flags=0: L.mx_gemm_ex(ctypes.byref(A), ctypes.byref(B), FAKE, 1, 64, flags, None)
    int8 = _t(mx, 4, 64, 256)
    fp6 = _t(mx, 6, 64, 256)
    nv = _t(mx, 3, 64, 256)
    assert g(int8, nv) == 5
    assert g(int8, fp6, 1) == 5
    tiled = mx._Tensor(4, 1, 64, 1024, FAKE, FAKE, None)
    assert g(tiled, tiled) == 5
    short = _t(mx, 6, 64, 224)
    assert g(int8, short) == 2


def test_other_entry_point_checks(mx):
    L = mx.load()
    rng = mx._Rng(0, 0)
    a8 = _t(mx, 1, 64, 64)
    a4 = _t(mx, 2, 64, 64)
    nv = _t(mx, 3, 64, 64)
    # gemm: a mixed pair with NVFP4, K mismatch, K % 32, C pitch
    assert L.mx_gemm(ctypes.byref(a8), ctypes.byref(nv), FAKE, 1, 64, None) == 5
    b = _t(mx, 1, 64, 96)
    assert L.mx_gemm(ctypes.byref(a8), ctypes.byref(b), FAKE, 1, 64, None) == 2
    assert L.mx_gemm(ctypes.byref(a8), ctypes.byref(a8), FAKE, 1, 63, None) == 2
    assert L.mx_gemm(ctypes.byref(a8), ctypes.byref(a8), None, 1, 64, None) == 1
    n16 = _t(mx, 3, 8, 48)
    assert L.mx_gemm(ctypes.byref(n16), ctypes.byref(n16), FAKE, 1, 8, None) == 2
    # grouped: non-NVFP4, groups < 1, rows not divisible, missing offsets
    assert L.mx_gemm_grouped(ctypes.byref(a8), None, 64, ctypes.byref(a8), 1, FAKE, FAKE, 0, 64, None) == 5
    assert L.mx_gemm_grouped(ctypes.byref(nv), None, 64, ctypes.byref(nv), 0, FAKE, FAKE, 0, 64, None) == 2
    assert L.mx_gemm_grouped(ctypes.byref(nv), None, 64, ctypes.byref(nv), 3, FAKE, FAKE, 0, 64, None) == 2
    assert L.mx_gemm_grouped(ctypes.byref(nv), None, 64, ctypes.byref(nv), 2, None, FAKE, 0, 32, None) == 1
    assert L.mx_gemm_grouped(ctypes.byref(nv), None, 60, ctypes.byref(nv), 2, FAKE, FAKE, 0, 32, None) == 2
    # grouped with a row gather but no A row to gather from
    nv0 = _t(mx, 3, 0, 64)
    assert L.mx_gemm_grouped(ctypes.byref(nv0), FAKE, 64, ctypes.byref(nv), 2, FAKE, FAKE, 0, 32, None) == 2
    # the products whose output is quantized need K > 0
    t0 = mx._Tensor(2, 1, 32, 0, None, None, None)
    q_out = _t(mx, 2, 32, 32)
    assert L.mx_gemm_quantize(ctypes.byref(t0), ctypes.byref(t0), ctypes.byref(q_out), 0, rng, 0, None) == 2
    b0 = _t(mx, 1, 64, 0, codes=None, scales=None)
    assert L.mx_gemm_quantize_a(FAKE, 64, 32, 1, 0, rng, ctypes.byref(b0), FAKE, 1, 64, None, None) == 2
    # requant: both or neither source, wrong out format, rows % 32
    out = _t(mx, 1, 64, 64)
    assert L.mx_requant_transpose(ctypes.byref(nv), FAKE, 64, 64, 64, ctypes.byref(out), 1, rng, None) == 1
    assert L.mx_requant_transpose(None, None, 64, 64, 64, ctypes.byref(out), 1, rng, None) == 1
    out4 = _t(mx, 2, 64, 64)
    assert L.mx_requant_transpose(ctypes.byref(nv), None, 0, 64, 64, ctypes.byref(out4), 1, rng, None) == 5
    assert L.mx_requant_transpose(None, FAKE, 64, 48, 64, ctypes.byref(out), 1, rng, None) == 2
    src8 = _t(mx, 1, 64, 64)
    assert L.mx_requant_transpose(ctypes.byref(src8), None, 0, 64, 64, ctypes.byref(out), 1, rng, None) == 5
    # hadamard: cols % 16, in-place with dtype change
    assert L.mx_hadamard16(FAKE, 0, FAKE, 0, 4, 24, 0, 0, None) == 2
    assert L.mx_hadamard16(FAKE, 0, FAKE, 1, 4, 32, 0, 0, None) == 5
    # amax / dequantize
    assert L.mx_amax(FAKE, 0, 4, 64, 64, 0, 0, None, None) == 1
    assert L.mx_amax(FAKE, 0, 4, 64, 64, 4, 0, FAKE, None) == 5
    assert L.mx_dequantize(ctypes.byref(a8), FAKE, 0, 32, 0, 0, None) == 2
    assert L.mx_dequantize(None, FAKE, 0, 64, 0, 0, None) == 1
    # error stats: missing output, cols % 8, pitch, unaligned output
    assert L.mx_error_stats(FAKE, 0, 64, FAKE, 64, 4, 64, None, None) == 1
    assert L.mx_error_stats(FAKE, 0, 64, FAKE, 64, 4, 60, FAKE, None) == 2
    assert L.mx_error_stats(FAKE, 0, 32, FAKE, 64, 4, 64, FAKE, None) == 2
    assert L.mx_error_stats(FAKE, 0, 64, FAKE, 64, 4, 64, ctypes.c_void_p(FAKE + 8), None) == 3
    # GEMM quantizing A in its prologue: missing B, A format, rounding mode, B
    # format, missing / unaligned A, A pitch, missing C, Q(A) format and shape
    f = L.mx_gemm_quantize_a
    assert f(FAKE, 64, 32, 1, 0, rng, None, FAKE, 1, 64, None, None) == 1
    assert f(FAKE, 64, 32, 3, 0, rng, ctypes.byref(a8), FAKE, 1, 64, None, None) == 5
    assert f(FAKE, 64, 32, 1, 2, rng, ctypes.byref(a8), FAKE, 1, 64, None, None) == 4
    assert f(FAKE, 64, 32, 1, 0, rng, ctypes.byref(nv), FAKE, 1, 64, None, None) == 5
    assert f(None, 64, 32, 1, 0, rng, ctypes.byref(a8), FAKE, 1, 64, None, None) == 1
    assert f(ctypes.c_void_p(FAKE + 8), 64, 32, 1, 0, rng, ctypes.byref(a8), FAKE, 1, 64, None, None) == 3
    assert f(FAKE, 48, 32, 1, 0, rng, ctypes.byref(a8), FAKE, 1, 64, None, None) == 2
    assert f(FAKE, 64, 32, 1, 0, rng, ctypes.byref(a8), None, 1, 64, None, None) == 1
    q4 = _t(mx, 2, 32, 64)
    assert f(FAKE, 64, 32, 1, 0, rng, ctypes.byref(a8), FAKE, 1, 64, ctypes.byref(q4), None) == 5
    q8 = _t(mx, 1, 48, 64)
    assert f(FAKE, 64, 32, 1, 0, rng, ctypes.byref(a8), FAKE, 1, 64, ctypes.byref(q8), None) == 2


def test_binding_fails_loudly_without_library(mx, monkeypatch):
    monkeypatch.setattr(mx, "_lib", None)
    monkeypatch.setattr(mx, "LIB_PATH", "/nonexistent/libmx.so")
    with pytest.raises(mx.MXError):
        mx.load()


def _tl(mx, fmt, rows, cols, layout, ts=FAKE):
    return mx._Tensor(fmt, layout, rows, cols, FAKE, FAKE, ts)


def test_layout_argument_checks(mx):
    L = mx.load()
    rng = mx._Rng(0, 0)
    q = lambda out, rows, cols: L.mx_quantize(FAKE, 0, rows, cols, cols, ctypes.byref(out), 0, rng, 0, 0, None, None)
    assert q(_tl(mx, 2, 32, 1024, 7), 32, 1024) == 4              # unknown layout
    assert q(_tl(mx, 2, 32, 512, 1), 32, 512) == 2                # tiled needs cols % 1024
    assert q(_tl(mx, 2, 48, 1024, 1), 48, 1024) == 2              # tiled needs rows % 32
    assert L.mx_quantize(FAKE, 0, 32, 1024, 1024, ctypes.byref(_tl(mx, 3, 32, 1024, 1)), 0, rng, 0, 0,
                         FAKE, None) == 5                          # NVFP4 has no tiled layout
    g = lambda a, b, flags=0: L.mx_gemm_ex(ctypes.byref(a), ctypes.byref(b), FAKE, 0, 64, flags, None)
    assert g(_tl(mx, 2, 64, 1024, 1), _tl(mx, 2, 64, 1024, 0)) == 5  # mixed layouts
    assert g(_tl(mx, 1, 64, 1024, 1), _tl(mx, 1, 64, 1024, 1)) == 5  # tiled MXFP8 needs native
    src = _tl(mx, 3, 64, 1024, 1)
    assert L.mx_requant_transpose(ctypes.byref(src), None, 0, 64, 1024, ctypes.byref(_tl(mx, 1, 1024, 64, 0)),
                                  1, rng, None) == 5
    assert L.mx_requant_transpose(None, FAKE, 1024, 1024, 1024, ctypes.byref(_tl(mx, 1, 1024, 1024, 1)),
                                  1, rng, None) == 5               # tiled requant output
