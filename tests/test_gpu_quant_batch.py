"""mx_quantize_batch against individual mx_quantize calls, bit for bit:
tile-layout jobs that share launches (more than one launch's worth, mixed
shapes, per-job random streams), and lists mixing in jobs that are launched on
their own (row layout, NVFP4, other input dtypes)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import microscaling_precision_gemm_amd as mx
    from tests.gpu_util import dev, host, to_gpu_bf16, to_gpu_f32


def _x(rows, cols, seed, f32=False):
    bits = W.normal_bf16(rows, cols, 1.0, seed, 100, outlier_entries=0.002, outlier_mult=40.0)
    if f32:
        return to_gpu_f32(W.bf16_bits_to_f32(bits))
    return to_gpu_bf16(bits)


def _job(x, fmt, layout, rnd=0, seed=0, counter=0, flags=0, mask=0, amax=None):
    out = mx.empty(fmt, x.shape[0], x.shape[1], device=dev(), layout=layout)
    return dict(x=x, out=out, rnd=rnd, seed=seed, counter=counter, flags=flags, sign_mask=mask, amax=amax)


def _single(j):
    out = mx.empty(j["out"].fmt, j["x"].shape[0], j["x"].shape[1], device=dev(), layout=j["out"].layout)
    amax = None
    if j["amax"] is not None:
        amax = torch.zeros(1, dtype=torch.float32, device=dev())
    mx.mx_quantize(j["x"], out, j["rnd"], j["seed"], j["counter"], j["flags"], j["sign_mask"], amax)
    return out


def _check(jobs):
    mx.mx_quantize_batch(jobs)
    singles = [_single(j) for j in jobs]
    torch.cuda.synchronize()
    for k, (j, s) in enumerate(zip(jobs, singles)):
        c, sc, ts = host(j["out"])
        c2, sc2, ts2 = host(s)
        assert np.array_equal(sc, sc2), f"job {k}: scales"
        assert np.array_equal(c, c2), f"job {k}: codes"
        if ts is not None:
            assert np.array_equal(ts, ts2), f"job {k}: tensor scale"


def test_two_tiled_mxfp4_operands():
    T = mx.MX_LAYOUT_TILED
    _check([_job(_x(4096, 4096, 1), 2, T), _job(_x(4096, 4096, 2), 2, T)])


@pytest.mark.parametrize("rnd,rht", [(0, False), (1, False), (1, True)])
def test_more_jobs_than_one_launch_mixed_shapes(rnd, rht):
    T = mx.MX_LAYOUT_TILED
    flags = mx.MX_FLAG_RHT16 if rht else 0
    shapes = [(32, 1024), (96, 2048), (256, 3072), (64, 1024), (128, 2048), (32, 4096)]
    jobs = [_job(_x(r, c, 10 + i), 1, T, rnd, 7 + i, 1000 * i, flags, mx.mx_rht_signs(i) if rht else 0)
            for i, (r, c) in enumerate(shapes)]
    _check(jobs)


def test_lists_with_jobs_launched_on_their_own():
    T, Rw = mx.MX_LAYOUT_TILED, mx.MX_LAYOUT_ROWS
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    jobs = [
        _job(_x(64, 1024, 20), 2, T),
        _job(_x(64, 1024, 21), 2, T, flags=mx.MX_FLAG_SCALE_CEIL),
        _job(_x(48, 512, 22), 1, Rw, rnd=1, seed=3),
        _job(_x(64, 1024, 23), 2, T),
        _job(_x(64, 512, 24), 3, Rw, amax=amax),
        _job(_x(64, 1024, 25, f32=True), 2, T),
        _job(_x(64, 1024, 26), 1, T),
        _job(_x(96, 2048, 27), 1, T),
    ]
    _check(jobs)


def test_empty_jobs_and_empty_list():
    mx.mx_quantize_batch([])
    T = mx.MX_LAYOUT_TILED
    z = torch.empty(0, 1024, dtype=torch.bfloat16, device=dev())
    _check([_job(z, 2, mx.MX_LAYOUT_ROWS), _job(_x(32, 1024, 30), 2, T)])


# --- NVFP4 jobs: one launch per pass for up to 16 compatible jobs --------------
def _nv(rows, cols, seed, rnd=0, flags=0, mask=0, counter=0, amax=None, f32=False):
    x = _x(rows, cols, seed, f32)
    a = amax if amax is not None else torch.zeros(1, dtype=torch.float32, device=dev())
    return _job(x, 3, mx.MX_LAYOUT_ROWS, rnd, seed, counter, flags, mask, amax=a)


NV_SHAPES = [(64, 1024), (33, 2048), (128, 512), (17, 4096), (256, 1040), (1, 160)]


@pytest.mark.parametrize("variant", ["rne", "sr", "rht_sr", "four6", "2d", "2d_sr", "f32"])
def test_nvfp4_jobs_share_launches(variant):
    """Several NVFP4 tensors (ragged rows and columns, per-job seeds and
    counters) through one batch: bit-identical to one mx_quantize call each,
    tensor scales included."""
    rnd = 1 if "sr" in variant else 0
    flags = {"rht_sr": mx.MX_FLAG_RHT16, "four6": mx.MX_FLAG_FOUR_OVER_SIX, "2d": mx.MX_FLAG_BLOCK_2D,
             "2d_sr": mx.MX_FLAG_BLOCK_2D}.get(variant, 0)
    mask = mx.mx_rht_signs(5) if variant == "rht_sr" else 0
    jobs = [_nv(r, c, 40 + i, rnd, flags, mask, counter=777 * i, f32=variant == "f32")
            for i, (r, c) in enumerate(NV_SHAPES)]
    _check(jobs)


def test_nvfp4_more_than_one_launch_and_expert_weights():
    """20 expert-weight slices of one stacked tensor (2-D blocks, each expert
    its own tensor-scale and amax slot, as a mixture-of-experts layer keeps
    them): two launches per pass, same results as 20 calls."""
    E, rows, cols = 20, 96, 1024
    W_ = _x(E * rows, cols, 60)
    q = mx.empty(3, E * rows, cols, device=dev(), n_tensor_scales=E)
    amax = torch.zeros(E, dtype=torch.float32, device=dev())
    jobs = [dict(x=W_[e * rows:(e + 1) * rows], out=q.view_rows(e * rows, (e + 1) * rows, q.tensor_scale[e:e + 1]),
                 rnd=0, seed=0, counter=0, flags=mx.MX_FLAG_BLOCK_2D, sign_mask=0, amax=amax[e:e + 1])
            for e in range(E)]
    _check(jobs)


def test_nvfp4_shared_amax_slot_keeps_call_order():
    """Jobs that name the same amax slot are not merged into one amax pass:
    each computes its own max, as consecutive calls do.  A slot given as input
    (MX_FLAG_AMAX_GIVEN) may be shared."""
    shared = torch.zeros(1, dtype=torch.float32, device=dev())
    a, b = _x(64, 1024, 70), _x(64, 1024, 71) * 3.0
    jobs = [_job(a, 3, mx.MX_LAYOUT_ROWS, amax=shared), _job(b, 3, mx.MX_LAYOUT_ROWS, amax=shared)]
    mx.mx_quantize_batch(jobs)
    torch.cuda.synchronize()
    for j in jobs:
        s = _single(j)
        torch.cuda.synchronize()
        assert np.array_equal(host(j["out"])[0], host(s)[0]) and np.array_equal(host(j["out"])[2], host(s)[2])
    given = torch.tensor([float(max(a.abs().max(), b.abs().max()))], dtype=torch.float32, device=dev())
    g = mx.MX_FLAG_AMAX_GIVEN
    jobs = [_job(a, 3, mx.MX_LAYOUT_ROWS, flags=g, amax=given), _job(b, 3, mx.MX_LAYOUT_ROWS, flags=g, amax=given)]
    mx.mx_quantize_batch(jobs)
    for j in jobs:
        out = mx.empty(3, 64, 1024, device=dev())
        mx.mx_quantize(j["x"], out, flags=g, amax=given)
        torch.cuda.synchronize()
        for u, v in zip(host(j["out"]), host(out)):
            assert np.array_equal(u, v)


def test_nvfp4_expert_weights_full_size_batch():
    """The mixture-of-experts weights at full size (32 experts of 2048 x 7168
    BF16, N(0, 0.02^2)), 2-D blocks, each expert its own amax and tensor scale,
    in one batch call as the benchmark runs it; experts 0 and 29 checked bit
    for bit against the oracle, tensor scales of all 32 against the oracle's
    T / 2688 of each expert."""
    import oracle
    E, rows, cols = 32, 2048, 7168
    bits = W.normal_bf16(E * rows, cols, 0.02, 0, 120)
    Wt = to_gpu_bf16(bits)
    q = mx.empty(3, E * rows, cols, device=dev(), n_tensor_scales=E)
    amax = torch.zeros(E, dtype=torch.float32, device=dev())
    jobs = [dict(x=Wt[e * rows:(e + 1) * rows], out=q.view_rows(e * rows, (e + 1) * rows, q.tensor_scale[e:e + 1]),
                 flags=mx.MX_FLAG_BLOCK_2D, amax=amax[e:e + 1]) for e in range(E)]
    mx.mx_quantize_batch(jobs)
    torch.cuda.synchronize()
    codes, scales, ts = host(q)
    for e in (0, 29):
        wc, ws, wts = oracle.quantize(bits[e * rows:(e + 1) * rows], 3, variant=oracle.V_2D)
        assert np.array_equal(scales[e * rows:(e + 1) * rows], ws), f"expert {e}: scales"
        assert np.array_equal(codes[e * rows:(e + 1) * rows], wc), f"expert {e}: codes"
        assert np.float32(ts[e]) == np.float32(wts), f"expert {e}: tensor scale"
    T = np.abs(W.bf16_bits_to_f32(bits).reshape(E, -1)).max(axis=1).astype(np.float32)
    assert np.array_equal(amax.cpu().numpy(), T)
    assert np.array_equal(ts.astype(np.float32), (T / np.float32(2688.0)).astype(np.float32))
