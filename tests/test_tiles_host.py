"""The host tile permutations against the layout's element-wise definition
(in include/mx.h), evaluated one element at a time on small arrays."""
import numpy as np

from tests.tiles import tile_codes, tile_scales, untile_codes, untile_scales


def test_code_tiles_match_definition():
    R, RB = 64, 256
    g = np.random.default_rng(0)
    codes = g.integers(0, 256, (R, RB), dtype=np.uint8)
    flat = tile_codes(codes).reshape(-1)
    for row in range(R):
        for kb in range(RB):
            T, r, t, c = row // 32, row % 32, kb // 128, (kb % 128) // 16
            off = (T * (RB // 128) + t) * 4096 + (c // 2) * 1024 + ((c % 2) * 32 + r) * 16 + kb % 16
            assert flat[off] == codes[row, kb]
    assert np.array_equal(untile_codes(tile_codes(codes), R, RB), codes)


def test_scale_tiles_match_definition():
    R, B = 64, 64  # cols = 2048
    g = np.random.default_rng(1)
    sc = g.integers(0, 256, (R, B), dtype=np.uint8)
    flat = tile_scales(sc).reshape(-1)
    for row in range(R):
        for blk in range(B):
            T, r, gi, b = row // 32, row % 32, blk // 32, blk % 32
            off = (T * (B // 32) + gi) * 1024 + ((b % 2) * 32 + r) * 16 + b // 2
            assert flat[off] == sc[row, blk]
    assert np.array_equal(untile_scales(tile_scales(sc), R, B), sc)
