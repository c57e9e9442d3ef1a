"""mx_quantize_batch_noalloc against mx_quantize_batch with caller-owned amax
slots, bit for bit, on two calls in a row: the second has fewer jobs and
smaller tensors whose amax lies far below what the first call left in the
library's slot array, so a slot that was read before being rewritten would
change the tensor scales.  Then the call recorded into a HIP graph (the use
it exists for): every replay, with an eager no-allocation call on other
inputs between replays, reproduces the eager result bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import dev, host, to_gpu_bf16, to_gpu_f32


def _x(rows, cols, seed, scale=1.0, f32=False):
    bits = W.normal_bf16(rows, cols, scale, seed, 300, outlier_entries=0.002, outlier_mult=40.0)
    if f32:
        return to_gpu_f32(W.bf16_bits_to_f32(bits))
    return to_gpu_bf16(bits)


def _jobs(specs):
    """specs: (x, fmt, layout, rnd, flags, seed) -> job dicts without amax."""
    out = []
    for x, fmt, layout, rnd, flags, seed in specs:
        o = mx.empty(fmt, x.shape[0], x.shape[1], device=dev(), layout=layout)
        mask = mx.mx_rht_signs(seed) if flags & mx.MX_FLAG_RHT16 else 0
        out.append(dict(x=x, out=o, rnd=rnd, seed=seed, counter=7 * seed, flags=flags, sign_mask=mask))
    return out


def _reference(jobs):
    """The same jobs through mx_quantize_batch, each NVFP4 job with its own
    caller-allocated amax slot."""
    ref = []
    for j in jobs:
        o = mx.empty(j["out"].fmt, j["x"].shape[0], j["x"].shape[1], device=dev(), layout=j["out"].layout)
        r = dict(j, out=o)
        if o.fmt == mx.MX_NVFP4:
            r["amax"] = torch.zeros(1, dtype=torch.float32, device=dev())
        ref.append(r)
    mx.mx_quantize_batch(ref)
    return ref


def _compare(jobs, ref):
    torch.cuda.synchronize()
    for k, (j, r) in enumerate(zip(jobs, ref)):
        c, sc, ts = host(j["out"])
        c2, sc2, ts2 = host(r["out"])
        assert np.array_equal(sc, sc2), f"job {k}: scales"
        assert np.array_equal(c, c2), f"job {k}: codes"
        if ts is not None:
            assert np.array_equal(ts, ts2), f"job {k}: tensor scale"


def _specs(n_nv, rows, cols, scale, seed0):
    T, R = mx.MX_LAYOUT_TILED, mx.MX_LAYOUT_ROWS
    variants = [(mx.MX_RNE, 0), (mx.MX_SR, mx.MX_FLAG_RHT16), (mx.MX_RNE, mx.MX_FLAG_BLOCK_2D),
                (mx.MX_RNE, mx.MX_FLAG_FOUR_OVER_SIX), (mx.MX_SR, 0)]
    specs = []
    for i in range(n_nv):
        rnd, flags = variants[(i // 4) % len(variants)]
        specs.append((_x(rows, cols, seed0 + i, scale), mx.MX_NVFP4, R, rnd, flags, seed0 + i))
    specs.append((_x(64, 1024, seed0 + 500, scale), mx.MX_MXFP4_E2M1, T, mx.MX_RNE, 0, 0))
    specs.append((_x(rows, cols, seed0 + 501, scale, f32=True), mx.MX_MXFP8_E4M3, R, mx.MX_SR, 0, 3))
    specs.append((_x(rows, cols, seed0 + 502, scale, f32=True), mx.MX_NVFP4, R, mx.MX_RNE, 0, 5))
    return specs


def test_noalloc_batch_matches_batch_on_two_calls():
    # first call: 70 NVFP4 jobs (more than one 64-job chunk) plus MX and FP32 jobs
    jobs = _jobs(_specs(70, 96, 512, 4.0, 1000))
    assert len(jobs) <= mx.MX_NOALLOC_MAX_JOBS
    mx.mx_quantize_batch_noalloc(jobs)
    _compare(jobs, _reference(jobs))
    # second call: fewer, smaller jobs with a 1000x smaller amax
    jobs2 = _jobs(_specs(9, 32, 256, 0.004, 2000))
    mx.mx_quantize_batch_noalloc(jobs2)
    _compare(jobs2, _reference(jobs2))


def test_noalloc_batch_rejects_what_it_cannot_hold():
    x = _x(32, 256, 9)
    jobs = _jobs([(x, mx.MX_NVFP4, mx.MX_LAYOUT_ROWS, mx.MX_RNE, 0, 1)] * (mx.MX_NOALLOC_MAX_JOBS + 1))
    with pytest.raises(mx.MXError):
        mx.mx_quantize_batch_noalloc(jobs)
    j = _jobs([(x, mx.MX_NVFP4, mx.MX_LAYOUT_ROWS, mx.MX_RNE, 0, 1)])
    j[0]["amax"] = torch.zeros(1, dtype=torch.float32, device=dev())
    with pytest.raises(mx.MXError):
        mx.mx_quantize_batch_noalloc(j)


def _graph_jobs(seed, scale):
    specs = [(mx.MX_RNE, 0), (mx.MX_SR, mx.MX_FLAG_RHT16), (mx.MX_RNE, mx.MX_FLAG_BLOCK_2D),
             (mx.MX_RNE, mx.MX_FLAG_FOUR_OVER_SIX), (mx.MX_SR, 0), (mx.MX_RNE, 0)]
    jobs = []
    for i, (rnd, flags) in enumerate(specs):
        x = to_gpu_bf16(W.normal_bf16(64, 512, scale * (i + 1), seed, 400 + i, outlier_entries=0.002,
                                      outlier_mult=30.0))
        mask = mx.mx_rht_signs(seed + i) if flags & mx.MX_FLAG_RHT16 else 0
        jobs.append(dict(x=x, out=mx.empty(mx.MX_NVFP4, 64, 512, dev()), rnd=rnd, seed=seed + i, counter=3 * i,
                         flags=flags, sign_mask=mask))
    x = to_gpu_bf16(W.normal_bf16(64, 1024, scale, seed, 420))
    jobs.append(dict(x=x, out=mx.empty(mx.MX_MXFP4_E2M1, 64, 1024, dev(), layout=mx.MX_LAYOUT_TILED)))
    return jobs


def _snap(jobs):
    return [tuple(np.copy(a) for a in host(j["out"]) if a is not None) for j in jobs]


def test_noalloc_batch_in_a_graph():
    jobs = _graph_jobs(1, 2.0)
    other = _graph_jobs(2, 0.001)
    qb = mx.QuantizeBatch(jobs, noalloc=True)
    qo = mx.QuantizeBatch(other, noalloc=True)
    qb.run()
    torch.cuda.synchronize()
    want = _snap(jobs)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qb.run()
    torch.cuda.synchronize()
    for rep in range(4):
        for j in jobs:
            j["out"].codes.fill_(0x5A)
            j["out"].scales.fill_(0x5A)
            if j["out"].tensor_scale is not None:
                j["out"].tensor_scale.fill_(-1.0)
        qo.run()  # other amax values into the shared slots
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snap(jobs)
        for k, (g, w) in enumerate(zip(got, want)):
            for a, b in zip(g, w):
                assert np.array_equal(a, b), f"replay {rep}, job {k}"
