"""Host check of the division replacement in the NVFP4 quantizers: the
block-scale quotient fl(a_b / d) is formed as the product a_b * fl(1/d)
corrected once by its exact residual (fused multiply-add), Markstein's
correction step.  Compared bit for bit with the FP32 division: every dividend
significand at two exponents for six divisors (including 2 - 2^-22 and 3) and
random dividend-divisor pairs whose quotient lies within a few units in the
last place of a rounding midpoint."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_corrected_quotient_equals_division():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "fdiv_check")
        # no contraction: each operation rounds as written
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                        os.path.join(HERE, "host", "fdiv_check.c"), "-lm"], check=True)
        out = subprocess.run([exe, "6", "20000000", "5"], check=True, capture_output=True,
                             text=True, timeout=300)
    assert int(out.stdout.strip()) == 0
