"""The C-ABI calls recorded into a HIP graph: every replay, with eager work
and synchronisations between replays, reproduces the eager results bit for
bit (codes, scales, tensor scale, GEMM output)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import dev, to_gpu_bf16


def _snap(*ts):
    out = []
    for t in ts:
        if isinstance(t, mx.MXTensor):
            out += [t.codes.cpu().numpy().copy(), t.scales.cpu().numpy().copy()]
            if t.tensor_scale is not None:
                out.append(t.tensor_scale.cpu().numpy().copy())
        else:
            out.append(t.cpu().numpy().copy() if t.dtype != torch.bfloat16 else t.view(torch.int16).cpu().numpy().copy())
    return out


def test_graph_replays_match_eager():
    M = N = 3072  # large enough for the pipelined GEMM kernel
    K = 512
    a = to_gpu_bf16(W.normal_bf16(M, K, 1.0, 0, 90, outlier_cols=0.01, outlier_mult=50))
    b = to_gpu_bf16(W.normal_bf16(N, K, 0.02, 0, 91))
    g = to_gpu_bf16(W.student_t_bf16(256, 512, 3.0, 0, 92))
    qa, qb = mx.empty(2, M, K, dev()), mx.empty(2, N, K, dev())
    qg = mx.empty(3, 256, 512, dev())
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    xt = mx.empty(1, 512, 256, dev())
    C = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    mask = mx.mx_rht_signs(3)

    def calls():
        mx.mx_quantize(a, qa)
        mx.mx_quantize(b, qb)
        mx.mx_gemm(qa, qb, C)
        mx.mx_quantize(g, qg, mx.MX_SR, 5, 11, mx.MX_FLAG_RHT16, mask, amax)
        mx.mx_requant_transpose(xt, src=qg, rnd=mx.MX_SR, seed=5, counter=99)

    calls()
    torch.cuda.synchronize()
    want = _snap(qa, qb, C, qg, xt)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    other = to_gpu_bf16(W.normal_bf16(M, K, 3.0, 1, 93))
    for rep in range(4):
        # clobber every output eagerly, then replay
        for t in (qa.codes, qa.scales, qb.codes, qb.scales, qg.codes, qg.scales, xt.codes, xt.scales):
            t.fill_(0x5A)
        C.fill_(float("nan"))
        mx.mx_quantize(other, qa)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snap(qa, qb, C, qg, xt)
        for i, (x, y) in enumerate(zip(got, want)):
            assert np.array_equal(x, y), f"replay {rep}: output {i} differs from eager"


def test_library_loaded_before_torch():
    """load() called before torch is imported still binds libmx.so to the HIP
    runtime torch uses (one runtime in the process): a quantization on
    torch's stream then runs and matches the oracle (in a fresh process)."""
    import os
    import subprocess
    import sys
    code = (
        "import microscaling_precision_gemm_amd as mx\n"
        "mx.load()\n"
        "import numpy as np, torch, oracle, workloads as W\n"
        "b = W.normal_bf16(64, 256, 1.0, 0, 5)\n"
        "x = torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)\n"
        "q = mx.empty(2, 64, 256, 'cuda')\n"
        "mx.mx_quantize(x, q)\n"
        "torch.cuda.synchronize()\n"
        "o = oracle.quantize(b, 2)\n"
        "assert np.array_equal(q.codes.cpu().numpy(), o[0]) and np.array_equal(q.scales.cpu().numpy(), o[1])\n"
        "print('ok')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]
