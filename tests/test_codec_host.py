"""The library's element encoders, decoders and Philox stream (the
__host__ __device__ code in csrc/device/codec.h), compiled for the host and
checked against the oracle: exhaustively for round-to-nearest-even over every
non-negative FP32 pattern up to +Inf (and a sample of negatives), on a
sample of values x random values (with the rounding thresholds) for
stochastic rounding, and on 32768 RNG draws."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_device_codecs_match_oracle_on_host(orc):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "codec_check")
    src = os.path.join(ROOT, "tests", "host_codec_check.cpp")
    inc = os.path.join(ROOT, "microscaling_precision_gemm_amd", "csrc")
    subprocess.run([hipcc, "-O2", "-x", "hip", "--offload-arch=gfx950", "-I", inc, src, "-o", exe,
                    "-ldl", "-lpthread"], check=True, capture_output=True)
    import oracle
    out = subprocess.run([exe, oracle.build(force=False)], capture_output=True, text=True,
                         timeout=600)
    assert out.returncode == 0 and out.stdout.strip().startswith("OK"), out.stdout + out.stderr
