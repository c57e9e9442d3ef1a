"""Host-side permutations between the row layout and the matrix-instruction
tile layout of MX code and scale arrays, written from the layout's
definition in include/mx.h (test infrastructure: used to compare tiled GPU
output with the row-major oracle and to upload oracle operands tiled)."""
import numpy as np


def tile_codes(codes: np.ndarray) -> np.ndarray:
    """[R, RB] row-major code bytes -> flat tiled bytes (R % 32 == 0,
    RB % 128 == 0)."""
    R, RB = codes.shape
    x = codes.reshape(R // 32, 32, RB // 128, 4, 2, 16)      # T, r, t, c//2, c%2, byte
    return np.ascontiguousarray(x.transpose(0, 2, 3, 4, 1, 5)).reshape(R, RB)


def untile_codes(tiled: np.ndarray, R: int, RB: int) -> np.ndarray:
    x = np.asarray(tiled).reshape(R // 32, RB // 128, 4, 2, 32, 16)  # T, t, c//2, c%2, r, byte
    return np.ascontiguousarray(x.transpose(0, 4, 1, 2, 3, 5)).reshape(R, RB)


def tile_scales(scales: np.ndarray) -> np.ndarray:
    """[R, B] row-major block scales (B = cols / 32, B % 32 == 0) -> tiled."""
    R, B = scales.shape
    x = scales.reshape(R // 32, 32, B // 32, 16, 2)            # T, r, g, b//2, b%2
    return np.ascontiguousarray(x.transpose(0, 2, 4, 1, 3)).reshape(R, B)


def untile_scales(tiled: np.ndarray, R: int, B: int) -> np.ndarray:
    x = np.asarray(tiled).reshape(R // 32, B // 32, 2, 32, 16)  # T, g, b%2, r, b//2
    return np.ascontiguousarray(x.transpose(0, 3, 1, 4, 2)).reshape(R, B)
