"""Python binding of libmx (block-scaled quantization and GEMM for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/mx.h``.  PyTorch provides
device memory and streams.  The functions keep the C names; tensors are
torch CUDA (HIP) tensors, results are written into caller-provided or newly
allocated torch buffers.  There is no CPU fallback: if ``libmx.so`` is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmx.so")

MX_MXFP8_E4M3, MX_MXFP4_E2M1, MX_NVFP4 = 1, 2, 3
MX_MXINT8, MX_MXFP8_E5M2, MX_MXFP6_E3M2, MX_MXFP6_E2M3 = 4, 5, 6, 7
MX_RNE, MX_SR = 0, 1
MX_BF16, MX_F32 = 0, 1
MX_FLAG_RHT16, MX_FLAG_AMAX_GIVEN = 1, 2
MX_FLAG_SCALE_CEIL, MX_FLAG_FOUR_OVER_SIX, MX_FLAG_BLOCK_2D = 4, 8, 16
MX_GEMM_FP8_NATIVE = 1
MX_LAYOUT_ROWS, MX_LAYOUT_TILED = 0, 1
MX_NOALLOC_MAX_JOBS = 256

FORMATS = {"mxfp8": MX_MXFP8_E4M3, "mxfp4": MX_MXFP4_E2M1, "nvfp4": MX_NVFP4, "mxint8": MX_MXINT8,
           "s2f6": MX_MXINT8, "mxfp8_e5m2": MX_MXFP8_E5M2, "mxfp6_e3m2": MX_MXFP6_E3M2,
           "mxfp6_e2m3": MX_MXFP6_E2M3}

# every function declared in include/mx.h
EXPORTED = [
    "mx_codes_bytes", "mx_scales_bytes", "mx_rht_signs", "mx_quantize", "mx_amax",
    "mx_dequantize", "mx_requant_transpose", "mx_hadamard16", "mx_gemm", "mx_gemm_ex",
    "mx_gemm_grouped", "mx_gemm_quantize", "mx_gemm_quantize_a", "mx_quantize_batch", "mx_error_stats",
    "mx_quantize_batch_noalloc", "mx_status_string",
]


class MXError(RuntimeError):
    pass


class _Tensor(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("layout", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class _Rng(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("counter", ctypes.c_uint64)]


class _Job(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("xdt", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld_x", ctypes.c_int64), ("out", ctypes.POINTER(_Tensor)),
                ("rnd", ctypes.c_int32), ("rng", _Rng), ("flags", ctypes.c_uint32),
                ("rht_sign_mask", ctypes.c_uint16), ("amax", ctypes.c_void_p)]


_lib = None


def load():
    """Load libmx.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MXError(f"{LIB_PATH} is not built; run microscaling_precision_gemm_amd.build.build()")
    # torch ships its own HIP runtime under the same soname.  Loaded first, it
    # is the one libmx.so binds to; loaded after libmx.so (which would pull in
    # the system copy), the process would hold two runtimes, and launches on
    # torch's streams would fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32, u64, u16 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint16)
    TP = ctypes.POINTER(_Tensor)
    sig = {
        "mx_codes_bytes": (ctypes.c_size_t, [i32, i64, i64]),
        "mx_scales_bytes": (ctypes.c_size_t, [i32, i64, i64]),
        "mx_rht_signs": (u16, [u64]),
        "mx_quantize": (i32, [vp, i32, i64, i64, i64, TP, i32, _Rng, u32, u16, vp, vp]),
        "mx_amax": (i32, [vp, i32, i64, i64, i64, u32, u16, vp, vp]),
        "mx_error_stats": (i32, [vp, i32, i64, vp, i64, i64, i64, vp, vp]),
        "mx_dequantize": (i32, [TP, vp, i32, i64, u32, u16, vp]),
        "mx_requant_transpose": (i32, [TP, vp, i64, i64, i64, TP, i32, _Rng, vp]),
        "mx_hadamard16": (i32, [vp, i32, vp, i32, i64, i64, u16, i32, vp]),
        "mx_gemm": (i32, [TP, TP, vp, i32, i64, vp]),
        "mx_gemm_ex": (i32, [TP, TP, vp, i32, i64, u32, vp]),
        "mx_gemm_grouped": (i32, [TP, vp, i64, TP, i32, vp, vp, i32, i64, vp]),
        "mx_gemm_quantize": (i32, [TP, TP, TP, i32, _Rng, u32, vp]),
        "mx_gemm_quantize_a": (i32, [vp, i64, i64, i32, i32, _Rng, TP, vp, i32, i64, TP, vp]),
        "mx_quantize_batch": (i32, [ctypes.POINTER(_Job), i32, vp]),
        "mx_quantize_batch_noalloc": (i32, [ctypes.POINTER(_Job), i32, vp]),
        "mx_status_string": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise MXError(f"libmx: {load().mx_status_string(status).decode()} (status {status})")


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MX_BF16
    if t.dtype == torch.float32:
        return MX_F32
    raise MXError(f"unsupported dtype {t.dtype}")


class MXTensor:
    """A quantized [rows, cols] matrix: codes, block scales and (NVFP4) the
    per-tensor scale, as torch uint8 / float32 device tensors; `layout` is
    MX_LAYOUT_ROWS or MX_LAYOUT_TILED (byte order specified in mx.h)."""

    def __init__(self, fmt: int, rows: int, cols: int, codes, scales, tensor_scale=None,
                 layout: int = MX_LAYOUT_ROWS):
        self.fmt, self.rows, self.cols = int(fmt), int(rows), int(cols)
        self.codes, self.scales, self.tensor_scale = codes, scales, tensor_scale
        self.layout = int(layout)

    def desc(self) -> _Tensor:
        return _Tensor(self.fmt, self.layout, self.rows, self.cols, _ptr(self.codes),
                       _ptr(self.scales), _ptr(self.tensor_scale))

    def view_rows(self, r0: int, r1: int, tensor_scale=None) -> "MXTensor":
        """Rows [r0, r1) as a tensor sharing storage (row layout only)."""
        if self.layout != MX_LAYOUT_ROWS:
            raise MXError("view_rows needs the row layout")
        return MXTensor(self.fmt, r1 - r0, self.cols, self.codes[r0:r1], self.scales[r0:r1],
                        tensor_scale if tensor_scale is not None else self.tensor_scale)


def empty(fmt: int, rows: int, cols: int, device="cuda", n_tensor_scales: int = 1,
          layout: int = MX_LAYOUT_ROWS) -> MXTensor:
    """Allocate the buffers of a quantized [rows, cols] tensor.  (Tiled
    tensors have the same byte counts; their [rows, bytes/rows] shape is
    only a container.)"""
    torch = _torch()
    L = load()
    cb = L.mx_codes_bytes(fmt, rows, cols)
    sb = L.mx_scales_bytes(fmt, rows, cols)
    codes = torch.empty((rows, cb // max(rows, 1)), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, sb // max(rows, 1)), dtype=torch.uint8, device=device)
    ts = torch.empty(n_tensor_scales, dtype=torch.float32, device=device) if fmt == MX_NVFP4 else None
    return MXTensor(fmt, rows, cols, codes, scales, ts, layout)


def mx_codes_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(load().mx_codes_bytes(fmt, rows, cols))


def mx_scales_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(load().mx_scales_bytes(fmt, rows, cols))


def mx_rht_signs(seed: int) -> int:
    return int(load().mx_rht_signs(seed))


def mx_quantize(x, out: MXTensor, rnd: int = MX_RNE, seed: int = 0, counter: int = 0,
                flags: int = 0, sign_mask: int = 0, amax=None, stream=None) -> MXTensor:
    """Quantize x [rows, cols] (bf16 or fp32, row pitch x.stride(0)) into `out`.
    NVFP4 needs `amax` (a 1-element fp32 device tensor): read when
    MX_FLAG_AMAX_GIVEN is set, else computed into it."""
    L = load()
    d = out.desc()
    _check(L.mx_quantize(_ptr(x), _dt(x), x.shape[0], x.shape[1], x.stride(0), ctypes.byref(d),
                         rnd, _Rng(seed, counter), flags, sign_mask, _ptr(amax), _stream(stream)))
    return out


class QuantizeBatch:
    """A prepared mx_quantize_batch call: the job array is built once (the
    tensors must stay alive), and each run() is one call of the C function."""

    def __init__(self, jobs, noalloc: bool = False):
        self._descs = [j["out"].desc() for j in jobs]
        self._keep = [j["x"] for j in jobs] + [j["out"] for j in jobs]
        self._arr = (_Job * max(len(jobs), 1))()
        for i, j in enumerate(jobs):
            x = j["x"]
            self._arr[i] = _Job(_ptr(x), _dt(x), x.shape[0], x.shape[1], x.stride(0),
                                ctypes.pointer(self._descs[i]), j.get("rnd", MX_RNE),
                                _Rng(j.get("seed", 0), j.get("counter", 0)), j.get("flags", 0),
                                j.get("sign_mask", 0), _ptr(j.get("amax")))
        self._n = len(jobs)
        L = load()
        self._fn = L.mx_quantize_batch_noalloc if noalloc else L.mx_quantize_batch

    def run(self, stream=None):
        _check(self._fn(self._arr, self._n, _stream(stream)))


def mx_quantize_batch(jobs, stream=None):
    """Several mx_quantize calls in one: each job is a dict with the keys of
    mx_quantize (x, out, and optionally rnd, seed, counter, flags, sign_mask,
    amax).  Compatible tile-layout jobs share kernel launches."""
    QuantizeBatch(jobs).run(stream)
    return [j["out"] for j in jobs]


def mx_quantize_batch_noalloc(jobs, stream=None):
    """mx_quantize_batch without an amax buffer from the caller: NVFP4 jobs
    take their amax slots from the library's own device array (no job may
    carry "amax" or MX_FLAG_AMAX_GIVEN; at most MX_NOALLOC_MAX_JOBS jobs)."""
    QuantizeBatch(jobs, noalloc=True).run(stream)
    return [j["out"] for j in jobs]


def mx_amax(x, amax, flags: int = 0, sign_mask: int = 0, stream=None):
    L = load()
    _check(L.mx_amax(_ptr(x), _dt(x), x.shape[0], x.shape[1], x.stride(0), flags, sign_mask,
                     _ptr(amax), _stream(stream)))
    return amax


def mx_dequantize(t: MXTensor, y, flags: int = 0, sign_mask: int = 0, stream=None):
    L = load()
    d = t.desc()
    _check(L.mx_dequantize(ctypes.byref(d), _ptr(y), _dt(y), y.stride(0), flags, sign_mask,
                           _stream(stream)))
    return y


def mx_error_stats(x, y, stats, stream=None):
    """Round-trip error statistics of the FP32 tensor y against x (bf16 or
    fp32, same shape) into `stats` (4 float64 on the device): sum (y-x)^2,
    sum x^2, sum (y-x), max |y-x|."""
    L = load()
    rows, cols = x.shape
    _check(L.mx_error_stats(_ptr(x), _dt(x), x.stride(0), _ptr(y), y.stride(0), rows, cols, _ptr(stats),
                            _stream(stream)))
    return stats


def mx_requant_transpose(out: MXTensor, src: MXTensor | None = None, x_bf16=None,
                         rnd: int = MX_SR, seed: int = 0, counter: int = 0, stream=None):
    """Source [rows, cols] (NVFP4 `src` or bf16 `x_bf16`) -> MXFP8 `out` of
    shape [cols, rows]."""
    L = load()
    sdesc = None
    if src is not None:
        rows, cols = src.rows, src.cols
        sdesc = src.desc()
        sd = ctypes.byref(sdesc)
        xp, ld = None, 0
    else:
        rows, cols = x_bf16.shape
        sd = None
        xp, ld = _ptr(x_bf16), x_bf16.stride(0)
    od = out.desc()
    _check(L.mx_requant_transpose(sd, xp, ld, rows, cols, ctypes.byref(od), rnd,
                                  _Rng(seed, counter), _stream(stream)))
    return out


def mx_hadamard16(x, y, sign_mask: int, inverse: bool = False, stream=None):
    L = load()
    _check(L.mx_hadamard16(_ptr(x), _dt(x), _ptr(y), _dt(y), x.shape[0], x.shape[1], sign_mask,
                           int(inverse), _stream(stream)))
    return y


def mx_gemm(A: MXTensor, B: MXTensor, C, stream=None):
    """C [M, N] (fp32 or bf16, row pitch C.stride(0)) = A [M, K] * B [N, K]^T."""
    L = load()
    da, db = A.desc(), B.desc()
    _check(L.mx_gemm(ctypes.byref(da), ctypes.byref(db), _ptr(C), _dt(C), C.stride(0),
                     _stream(stream)))
    return C


def mx_gemm_ex(A: MXTensor, B: MXTensor, C, flags: int = 0, stream=None):
    """mx_gemm with options (MX_GEMM_FP8_NATIVE: MXFP8 on the FP8 matrix
    instruction, see include/mx.h for its accuracy)."""
    L = load()
    da, db = A.desc(), B.desc()
    _check(L.mx_gemm_ex(ctypes.byref(da), ctypes.byref(db), _ptr(C), _dt(C), C.stride(0), flags,
                        _stream(stream)))
    return C


def mx_gemm_quantize(A: MXTensor, B: MXTensor, out: MXTensor, rnd: int = MX_RNE, seed: int = 0,
                     counter: int = 0, flags: int = 0, stream=None) -> MXTensor:
    """C = A * B^T (tile-layout MX operands) written quantized into `out`
    (MXFP8 or MXFP4, [M, N], row or tile layout) by the GEMM's epilogue.
    flags: MX_GEMM_FP8_NATIVE (MXFP8 operands), MX_FLAG_SCALE_CEIL."""
    L = load()
    da, db, do = A.desc(), B.desc(), out.desc()
    _check(L.mx_gemm_quantize(ctypes.byref(da), ctypes.byref(db), ctypes.byref(do), rnd,
                              _Rng(seed, counter), flags, _stream(stream)))
    return out


def mx_gemm_quantize_a(A, a_fmt: int, B: MXTensor, C, rnd: int = MX_RNE, seed: int = 0, counter: int = 0,
                       a_out: "MXTensor | None" = None, stream=None):
    """C = Q(A) * B^T with A a BF16 [M, K] matrix quantized to a_fmt (MXFP8
    E4M3 or MXFP4) inside the GEMM; Q(A) also lands in a_out when given."""
    L = load()
    db = B.desc()
    dq = a_out.desc() if a_out is not None else None
    _check(L.mx_gemm_quantize_a(_ptr(A), A.stride(0), A.shape[0], a_fmt, rnd, _Rng(seed, counter),
                                ctypes.byref(db), _ptr(C), _dt(C), C.stride(0),
                                ctypes.byref(dq) if dq is not None else None, _stream(stream)))
    return C


def mx_gemm_grouped(A: MXTensor, row_index, routed_rows: int, B: MXTensor, num_groups: int,
                    group_offsets, C, stream=None):
    L = load()
    da, db = A.desc(), B.desc()
    _check(L.mx_gemm_grouped(ctypes.byref(da), _ptr(row_index), routed_rows, ctypes.byref(db),
                             num_groups, _ptr(group_offsets), _ptr(C), _dt(C), C.stride(0),
                             _stream(stream)))
    return C
