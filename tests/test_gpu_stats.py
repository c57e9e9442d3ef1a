"""GPU round-trip error statistics (mx_error_stats) of the RHT + NVFP4 codec
against the oracle's: the gradient tensor of the pages' fourth workload shape
(Student-t, nu = 3), quantized with round-to-nearest or stochastic rounding,
with or without the 16-point Hadamard transform, decoded (the inverse
transform applied when it was used) and compared with its source.  The GPU
chain is quantize -> dequantize -> statistics, all on the device; the oracle
side is the oracle's quantizer, decoder and inverse transform, and the plain
FP64 sums of oracle.roundtrip_stats."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import dev, to_gpu_bf16


def _gpu_chain(bits, rnd, rht, mask, seed=0):
    rows, cols = bits.shape
    x = to_gpu_bf16(bits)
    q = mx.empty(mx.MX_NVFP4, rows, cols, device=dev())
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    mx.mx_quantize(x, q, rnd, seed, 0, mx.MX_FLAG_RHT16 if rht else 0, mask, amax)
    y = torch.empty(rows, cols, dtype=torch.float32, device=dev())
    mx.mx_dequantize(q, y, mx.MX_FLAG_RHT16 if rht else 0, mask)
    st = torch.empty(4, dtype=torch.float64, device=dev())
    mx.mx_error_stats(x, y, st)
    torch.cuda.synchronize()
    return st.cpu().numpy()


def _oracle_chain(bits, rnd, rht, mask, seed=0):
    rows, cols = bits.shape
    c, s, S = oracle.quantize(bits, oracle.NVFP4, rnd, seed, 0, rht=rht, sign_mask=mask)
    y = oracle.dequantize(oracle.NVFP4, c, s, S, rows, cols)
    if rht:
        y = oracle.rht16(y, mask, inverse=True)
    return np.array(oracle.roundtrip_stats(bits, y)), y


def _compare(got, want, y, bits, what):
    d_abs = float(np.sum(np.abs(np.asarray(y, np.float64) - oracle.bf16_bits_to_f64(bits))))
    assert abs(got[0] - want[0]) <= 1e-12 * want[0], what
    assert abs(got[1] - want[1]) <= 1e-12 * want[1], what
    assert abs(got[2] - want[2]) <= 1e-12 * d_abs, what
    assert got[3] == want[3], what


@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("rht", [False, True])
def test_error_stats_match_the_oracle(rnd, rht):
    bits = W.student_t_bf16(512, 7168, 3.0, 0, 10)
    mask = mx.mx_rht_signs(0)
    got = _gpu_chain(bits, rnd, rht, mask)
    want, y = _oracle_chain(bits, rnd, rht, mask)
    _compare(got, want, y, bits, f"rnd={rnd} rht={rht}")


def test_error_stats_full_size():
    """All four combinations on the full 8192 x 7168 gradient tensor, against
    the oracle.  With the same block scales (they do not depend on the
    rounding), stochastic rounding never lands nearer than round-to-nearest,
    so its relative RMSE is the larger one."""
    bits = W.student_t_bf16(8192, 7168, 3.0, 0, 10)
    mask = mx.mx_rht_signs(0)
    rel = {}
    for rnd in (0, 1):
        for rht in (False, True):
            got = _gpu_chain(bits, rnd, rht, mask)
            want, y = _oracle_chain(bits, rnd, rht, mask)
            _compare(got, want, y, bits, f"full rnd={rnd} rht={rht}")
            rel[(rnd, rht)] = (np.sqrt(got[0] / got[1]), got[2] / bits.size)
    assert rel[(1, False)][0] > rel[(0, False)][0] and rel[(1, True)][0] > rel[(0, True)][0]


def test_error_stats_fp32_input_and_pitch():
    """FP32 source with a row pitch, against the oracle's plain sums."""
    g = np.random.default_rng(4)
    x = g.standard_normal((64, 96)).astype(np.float32)
    y = (x + g.standard_normal(x.shape).astype(np.float32) * 1e-3).astype(np.float32)
    xf = torch.zeros(64, 104, dtype=torch.float32, device=dev())
    xf[:, :96] = torch.from_numpy(x)
    yf = torch.zeros(64, 112, dtype=torch.float32, device=dev())
    yf[:, :96] = torch.from_numpy(y)
    st = torch.empty(4, dtype=torch.float64, device=dev())
    mx.mx_error_stats(xf[:, :96], yf[:, :96], st)
    torch.cuda.synchronize()
    got = st.cpu().numpy()
    want = oracle.roundtrip_stats(x, y)
    assert abs(got[0] - want[0]) <= 1e-12 * want[0] and abs(got[1] - want[1]) <= 1e-12 * want[1]
    assert abs(got[2] - want[2]) <= 1e-12 * float(np.sum(np.abs(y.astype(np.float64) - x))) and got[3] == want[3]
