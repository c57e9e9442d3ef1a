"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no quantization or GEMM arithmetic: it only draws random
matrices and routing tables.  Both the HIP path and the CPU oracle consume
the bytes it returns.

Recipe (every workload):
  * generator: numpy ``Generator(PCG64(SeedSequence([seed, tensor_id])))``;
  * draws are FP64, rounded to FP32 (numpy cast), then to BF16 with
    round-to-nearest-even on the bit pattern; BF16 data is returned as the
    raw ``uint16`` bit patterns;
  * outliers: ``k = round(fraction * count)`` distinct seeded positions
    (entries) or columns, multiplied in FP64 before rounding.

The five workloads mirror the shapes, distributions and outlier structure of
the pages' setting (MoE training in NVFP4 forward / MXFP8 backward; see
"Thinking Machines ... Inkling 2 Small" and "Microscaling (MX) and
block-scaled 4-bit formats"); no dataset is involved.
"""
from __future__ import annotations

import numpy as np


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id])))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """FP64 -> FP32 (numpy, RNE) -> BF16 bits (RNE on the FP32 pattern)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    b = (b + 0x7FFF + lsb) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rows: int, cols: int, std: float = 1.0, seed: int = 0, tensor_id: int = 0,
                outlier_entries: float = 0.0, outlier_cols: float = 0.0,
                outlier_mult: float = 1.0) -> np.ndarray:
    g = rng(seed, tensor_id)
    x = g.standard_normal((rows, cols)) * std
    if outlier_entries > 0:
        k = int(round(outlier_entries * rows * cols))
        pos = g.choice(rows * cols, size=k, replace=False)
        x.reshape(-1)[pos] *= outlier_mult
    if outlier_cols > 0:
        k = int(round(outlier_cols * cols))
        cidx = g.choice(cols, size=k, replace=False)
        x[:, cidx] *= outlier_mult
    return f64_to_bf16_bits(x)


def student_t_bf16(rows: int, cols: int, nu: float = 3.0, seed: int = 0,
                   tensor_id: int = 0) -> np.ndarray:
    g = rng(seed, tensor_id)
    return f64_to_bf16_bits(g.standard_t(nu, size=(rows, cols)))


def uniform_topk_routing(tokens: int, experts: int, topk: int, seed: int = 0, tensor_id: int = 9):
    """Each token picks ``topk`` distinct experts uniformly at random.

    Returns (row_index, group_offsets): routed rows sorted by expert (stable
    in token order), ``row_index[r]`` the token of routed row r, and
    ``group_offsets`` [experts + 1] (int64) delimiting each expert's rows."""
    g = rng(seed, tensor_id)
    keys = g.random((tokens, experts))
    choice = np.argsort(keys, axis=1, kind="stable")[:, :topk]  # distinct, uniform
    tok = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    exp = choice.reshape(-1).astype(np.int64)
    order = np.lexsort((tok, exp))
    row_index = tok[order].astype(np.int32)
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    return row_index, offsets


# --- the five workloads ----------------------------------------------------
def cfg1(seed: int = 0):
    """MXFP8 E4M3 RNE quantize of A, B 256x256 N(0,1) with 0.1% entries x100,
    then the 256^3 block-scaled GEMM to FP32."""
    A = normal_bf16(256, 256, 1.0, seed, 1, outlier_entries=0.001, outlier_mult=100.0)
    B = normal_bf16(256, 256, 1.0, seed, 2, outlier_entries=0.001, outlier_mult=100.0)
    return A, B


def cfg2(seed: int = 0, n: int = 4096):
    """MXFP4 E2M1 quantize + GEMM n^3: activations N(0,1) with 1% of the
    K-columns x50, weights N(0, 0.02^2); RNE; BF16 out."""
    A = normal_bf16(n, n, 1.0, seed, 3, outlier_cols=0.01, outlier_mult=50.0)
    B = normal_bf16(n, n, 0.02, seed, 4)
    return A, B


def cfg3(seed: int = 0, tokens: int = 4096, hidden: int = 7168, experts: int = 32,
         topk: int = 8, inter: int = 2048):
    """NVFP4 forward grouped GEMM: activations [tokens, hidden] N(0,1), top-k
    uniform routing, per-expert weights [inter, hidden] N(0, 0.02^2)."""
    X = normal_bf16(tokens, hidden, 1.0, seed, 5)
    row_index, offsets = uniform_topk_routing(tokens, experts, topk, seed, 6)
    W = [normal_bf16(inter, hidden, 0.02, seed, 100 + e) for e in range(experts)]
    return X, row_index, offsets, W


def cfg4(seed: int = 0, tokens: int = 16384, hidden: int = 4096, out: int = 14336):
    """Backward requant: X [tokens, hidden] N(0,1) with 0.5% entries x30
    (quantized to NVFP4 as setup), dY [tokens, out] N(0,1)."""
    X = normal_bf16(tokens, hidden, 1.0, seed, 7, outlier_entries=0.005, outlier_mult=30.0)
    dY = normal_bf16(tokens, out, 1.0, seed, 8)
    return X, dY


def cfg5(seed: int = 0, rows: int = 8192, cols: int = 7168):
    """Gradient tensor [rows, cols] Student-t(nu = 3) for RHT16 + NVFP4 SR."""
    return student_t_bf16(rows, cols, 3.0, seed, 10)
