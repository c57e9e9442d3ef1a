"""Pins for the oracle's counter-based generator (Philox-4x32-10).

The independent reference is rocRAND's Philox-4x32-10 engine (an installed
header-only library, compiled here for the host and run, not read into the
oracle): seeding it with key = seed and skipping 4*c outputs makes its next
four outputs the block function at counter (c_lo, c_hi, 0, 0).
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

HOST_PROG = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  for (int i = 1; i + 1 < argc; i += 2) {
    unsigned long long seed = strtoull(argv[i], 0, 0);
    unsigned long long c = strtoull(argv[i + 1], 0, 0);
    rocrand_device::philox4x32_10_engine e(seed, 0, 4ULL * c);
    unsigned a = e.next(), b = e.next(), d = e.next(), f = e.next();
    printf("%u %u %u %u\n", a, b, d, f);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_ref():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("hipcc / rocRAND headers not available")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "ref.cpp")
    exe = os.path.join(d, "ref")
    open(src, "w").write(HOST_PROG)
    subprocess.run([hipcc, "-O1", src, "-o", exe], check=True, capture_output=True)

    def run(pairs):
        args = [exe]
        for s, c in pairs:
            args += [str(s), str(c)]
        out = subprocess.run(args, check=True, capture_output=True, text=True).stdout
        return [[int(t) for t in line.split()] for line in out.strip().splitlines()]

    return run


def test_philox_matches_rocrand(orc, rocrand_ref):
    g = np.random.default_rng(11)
    # the engine skips 4*c outputs with a 64-bit offset, so c < 2^62 here
    pairs = [(0, 0), (1, 0), (0, 1), (2**64 - 1, 2**62 - 1), (0x0123456789ABCDEF, 5),
             (7, 2**32 - 1), (7, 2**32)]
    pairs += [(int(s), int(c)) for s, c in zip(g.integers(0, 2**63, 40), g.integers(0, 2**62, 40))]
    ref = rocrand_ref(pairs)
    for (s, c), r in zip(pairs, ref):
        ours = orc.philox4x32_10([c & 0xFFFFFFFF, c >> 32, 0, 0], [s & 0xFFFFFFFF, s >> 32])
        assert ours == r, (s, c)


def test_rand16_layout(orc):
    """Element n of a stream takes 16-bit half (n & 1) of word (n & 7) >> 1 of
    call counter + n // 8."""
    seed, counter = 0xDEADBEEF12345678, 77
    for n in range(0, 64):
        c = counter + n // 8
        w = orc.philox4x32_10([c & 0xFFFFFFFF, c >> 32, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
        word = w[(n & 7) >> 1]
        assert orc.rand16(seed, counter, n) == (word >> (16 * (n & 1))) & 0xFFFF
    # 64-bit counter addition carries into the high word
    c = 2**32 - 1
    a = orc.rand16(1, c, 8)
    w = orc.philox4x32_10([0, 1, 0, 0], [1, 0])
    assert a == w[0] & 0xFFFF


def test_rand16_uniformity(orc):
    """Light statistical check: 16-bit values are uniform (chi-square over 256
    bins) and each bit is balanced."""
    n = 1 << 17
    vals = np.array([orc.rand16(3, 0, i) for i in range(n)], np.int64)
    hist = np.bincount(vals >> 8, minlength=256)
    exp = n / 256
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 256 + 6 * np.sqrt(2 * 256)
    for b in range(16):
        frac = ((vals >> b) & 1).mean()
        assert abs(frac - 0.5) < 5 * 0.5 / np.sqrt(n)


def test_rht_signs_from_reserved_counter(orc):
    for seed in (0, 1, 12345):
        w = orc.philox4x32_10([0, 0, 0, 1], [seed & 0xFFFFFFFF, seed >> 32])
        assert orc.rht_signs(seed) == w[0] & 0xFFFF
