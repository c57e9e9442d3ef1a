"""Helpers shared by the GPU parity tests (marshalling only; no method
arithmetic beyond the oracle calls)."""
import numpy as np
import torch

import oracle
import microscaling_precision_gemm_amd as mx


def dev():
    return torch.device("cuda:0")


def to_gpu_bf16(bits: np.ndarray, pad_cols: int = 0) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor; pad_cols > 0 gives a
    row pitch larger than the column count (returns a strided view)."""
    rows, cols = bits.shape
    full = np.zeros((rows, cols + pad_cols), np.uint16)
    full[:, :cols] = bits
    t = torch.from_numpy(full.view(np.int16)).to(dev()).view(torch.bfloat16)
    return t[:, :cols]


def to_gpu_f32(x: np.ndarray, pad_cols: int = 0) -> torch.Tensor:
    rows, cols = x.shape
    full = np.zeros((rows, cols + pad_cols), np.float32)
    full[:, :cols] = x
    return torch.from_numpy(full).to(dev())[:, :cols]


def bf16_bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def quantize_gpu(x: torch.Tensor, fmt, rnd=mx.MX_RNE, seed=0, counter=0, rht=False, mask=0,
                 amax_value=None):
    rows, cols = x.shape
    out = mx.empty(fmt, rows, cols, device=dev())
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    flags = mx.MX_FLAG_RHT16 if rht else 0
    if amax_value is not None:
        amax.fill_(amax_value)
        flags |= mx.MX_FLAG_AMAX_GIVEN
    mx.mx_quantize(x, out, rnd, seed, counter, flags, mask,
                   amax if fmt == mx.MX_NVFP4 else None)
    torch.cuda.synchronize()
    return out, amax


def host(t: mx.MXTensor):
    ts = None if t.tensor_scale is None else t.tensor_scale.cpu().numpy()
    return t.codes.cpu().numpy(), t.scales.cpu().numpy(), ts


def upload(fmt, codes: np.ndarray, scales: np.ndarray, ts=None) -> mx.MXTensor:
    rows = codes.shape[0]
    cols = codes.shape[1] * (1 if fmt == mx.MX_MXFP8_E4M3 else 2)
    t = mx.MXTensor(fmt, rows, cols, torch.from_numpy(np.ascontiguousarray(codes)).to(dev()),
                    torch.from_numpy(np.ascontiguousarray(scales)).to(dev()),
                    None if ts is None else torch.tensor(np.atleast_1d(np.asarray(ts, np.float32)),
                                                         device=dev()))
    return t


def check_gemm(C: np.ndarray, Chat: np.ndarray, tol: np.ndarray, bf16_out: bool, what=""):
    """C must be the output format's rounding of a value within the bound:
    FP32 output: C in [fp32_rne(Chat - tol), fp32_rne(Chat + tol)] (the plain
    |C - Chat| <= tol wherever Chat +- tol are FP32 values); BF16 output: C in
    [bf16_rne(Chat - tol), bf16_rne(Chat + tol)].  Where the oracle's value is
    NaN (a NaN scale code), C must be NaN, and nowhere else."""
    C = C.astype(np.float64)
    Chat = np.asarray(Chat, np.float64)
    nan_want = np.isnan(Chat)
    if bf16_out:
        lo, hi = oracle.bf16_interval(np.where(nan_want, 0.0, Chat), np.where(nan_want, 0.0, tol))
    else:
        lo, hi = oracle.f32_interval(np.where(nan_want, 0.0, Chat), np.where(nan_want, 0.0, tol))
    inside = (C >= lo) & (C <= hi)
    bad = np.where(nan_want, ~np.isnan(C), ~inside)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        msg = "; ".join(f"{tuple(i)}: got {C[tuple(i)]!r} want {Chat[tuple(i)]!r} tol {tol[tuple(i)]!r}"
                        for i in idx)
        ok = ~nan_want & ~np.isnan(C)
        ratio = np.max(np.abs(C - Chat)[ok] / np.maximum(tol[ok] / 1e-5, 1e-300)) if ok.any() else float("nan")
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance "
                             f"(max |err|/sum|ab| = {ratio:.3g}); {msg}")
