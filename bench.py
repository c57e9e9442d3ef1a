"""Benchmark of the block-scaled quantize + GEMM hot path on one MI355X.

One step = quantize A (activations 4096x4096 BF16, N(0,1), 1% of K-columns
x50) and B (weights 4096x4096 BF16, N(0, 0.02^2)) to MXFP4 E2M1 with E8M0
scales per 32 (round-to-nearest-even), then the block-scaled GEMM
C = A * B^T (4096^3, FP32 accumulation, BF16 out).  Inputs are resident in
HBM before the timed region and rotate over 16 copies (1 GiB of BF16) so the
256 MB last-level cache does not hold them between steps.  The quantizer
writes the matrix-instruction tile layout, which the GEMM reads with
register-direct loads.  The step's three calls are launched eagerly (--graph replays them from a HIP graph captured
once per input slot instead).

Prints one JSON line: metric / value (TFLOP/s of the whole step: 2*M*N*K per
step time), the roofline of the dominant kernel (the GEMM) measured with HIP
events on the stream the kernels run on, the quantizer's HBM throughput, a
CPU baseline (the oracle on a bounded sample, rank 0), and secondary
measurements of the other workloads (MXFP8 GEMM, NVFP4 grouped MoE GEMM,
backward requant + wgrad, RHT + NVFP4 stochastic rounding) unless
--no-detail is given.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense peaks (AMD public figures) and HBM bandwidth
PEAK_TFLOPS = {"fp4": 10100.0, "fp6": 10100.0, "fp8": 5000.0, "bf16": 2500.0}
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-detail", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a HIP graph captured through the C ABI "
                         "instead of launching its calls eagerly")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="output rows of the GEMM sample the oracle is timed on")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device copy (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


# HBM traffic of the GEMM kernel from the rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes, stored with the hash of the kernel source they were taken on: a
# changed kernel reports null until the counters are taken again.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_mxfp4_4096_traffic.txt")
# the headline GEMM's source and every header it includes: the traffic figure
# is used only while their combined hash matches the one it was measured on
_CSRC = os.path.join(ROOT, "microscaling_precision_gemm_amd", "csrc")
GEMM_SOURCES = [os.path.join(_CSRC, *p.split("/")) for p in (
    "kernels/gemm_tiled.hip", "device/codec.h", "device/cvt.h", "device/gemm_common.h", "device/lowscale.h",
    "device/mxenc.h", "device/wave.h", "launch.h")]


def gemm_traffic():
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    sha = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(p, "rb") as f:
            sha.update(f.read())
    h = sha.hexdigest()
    if kv.get("kernel_source_sha256") != h or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


class Timer:
    """Per-launch HIP-event timing on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) if self.pairs else float("nan")


def time_fn(torch, fn, iters, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(iters):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ts]))


def upload_bf16(torch, bits: np.ndarray):
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def headline(torch, mx, W, args):
    """Timed region: `steps` steps of eager launches (quantize A and B in one
    batched call -- one kernel launch for both operands -- then the GEMM), or
    with --graph replays of one HIP graph per input slot captured through the
    C ABI.  Then the kernel-timing region: the same calls
    launched eagerly, each bracketed by HIP events on the stream they run on
    (events between the launches of the timed region would stall it)."""
    M = N = K = 4096
    A_bits, B_bits = W.cfg2(0, 4096)
    A0 = upload_bf16(torch, A_bits)
    B0 = upload_bf16(torch, B_bits)
    nrot = 16
    As = [A0] + [A0.clone() for _ in range(nrot - 1)]
    Bs = [B0] + [B0.clone() for _ in range(nrot - 1)]
    # operands quantized straight into the matrix-instruction tile layout,
    # which the register-direct GEMM kernel reads
    qa = mx.empty(mx.MX_MXFP4_E2M1, M, K, layout=mx.MX_LAYOUT_TILED)
    qb = mx.empty(mx.MX_MXFP4_E2M1, N, K, layout=mx.MX_LAYOUT_TILED)
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")

    # one prepared batch per input slot: both operands quantized by one launch
    batches = [mx.QuantizeBatch([dict(x=As[i], out=qa), dict(x=Bs[i], out=qb)]) for i in range(nrot)]

    def launch(i):
        batches[i].run()
        mx.mx_gemm(qa, qb, C)

    for i in range(nrot):
        launch(i)
    torch.cuda.synchronize()
    graphs = None
    if args.graph:
        graphs = []
        for i in range(nrot):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                launch(i)
            graphs.append(g)
        torch.cuda.synchronize()

    def step(i):
        if graphs is not None:
            graphs[i % nrot].replay()
        else:
            launch(i % nrot)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # kernel timing: back-to-back launches of one kernel between two events
    # (per launch: the interval / count, launch gaps included, so a little
    # above the kernel's own duration); and every launch between its own pair
    # of events (which stalls the queue between launches and lets the clock
    # drop on some boxes: reported beside it, not used)
    nb = max(args.steps, 20)

    def batch_ms(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(nb):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / nb

    # The GEMM's share of a step: a batch of whole steps (quantize batch, then
    # GEMM, inputs rotating as in the timed region) minus the batch of the
    # quantize launches alone measured right after it, five such pairs, the
    # median difference.  The clock under sustained matrix work drifts by
    # ~10% over milliseconds, so the two batches of a pair are taken back to
    # back.  Back-to-back GEMMs with nothing between them run slower still
    # (the matrix unit never idles and the clock settles lower); that figure
    # is taken last and reported beside it, not used for the roofline.
    pairs = []
    for _ in range(5):
        sb = batch_ms(lambda i=0: launch(i % nrot))
        qb_ = batch_ms(lambda i=0: batches[i % nrot].run())
        pairs.append((sb - qb_, sb, qb_))
    pairs.sort()
    gemm_ms, step_batch_ms, quant_batch_ms = pairs[len(pairs) // 2]
    quant_ms = float(np.median([q for _, _, q in pairs])) / 2  # per operand: one launch quantizes both
    gemm_b2b_ms = batch_ms(lambda i=0: mx.mx_gemm(qa, qb, C))
    tq, tg = Timer(torch), Timer(torch)
    for i in range(args.steps):
        s = tq.start()
        batches[i % nrot].run()
        tq.stop(s)
        s = tg.start()
        mx.mx_gemm(qa, qb, C)
        tg.stop(s)
    torch.cuda.synchronize()
    flops = 2.0 * M * N * K
    # algorithmic bytes of one MXFP4 quantize of a 4096x4096 BF16 operand:
    # read 2 B/elem, write 0.5 B codes + 1/32 B scales
    qbytes = M * K * (2 + 0.5 + 1 / 32)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    out = {
        "ms_per_step": ms_step,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "gemm_ms": gemm_ms,
        "gemm_ms_back_to_back": gemm_b2b_ms,
        "step_batch_ms": step_batch_ms,
        "gemm_ms_bracketed": tg.mean_ms(),
        "quant_ms_bracketed": tq.mean_ms() / 2,
        "gemm_tflops": gemm_tflops,
        "quant_ms": quant_ms,
        "quant_gbs": qbytes / (quant_ms * 1e-3) / 1e9,
        "qbytes": qbytes,
        "flops": flops,
        "A_bits": A_bits,
        "B_bits": B_bits,
        "launch": "eager" if graphs is None else "hip graph per step",
    }
    return out


def cpu_baseline(W, oracle, A_bits, B_bits, rows: int, min_seconds: float = 10.0):
    """The oracle, untuned, on a bounded sample of the same step: quantize
    `rows` rows of A and all of B, then `rows` output rows of the FP64 GEMM,
    repeated until at least `min_seconds` have passed.  Throughput is reported
    in the step's unit (TFLOP/s of 2*M*N*K-equivalent work) over the sampled
    fraction of the output."""
    oracle.lib()
    threads = oracle.get_threads()
    M, K = A_bits.shape
    N = B_bits.shape[0]

    def run(r, nb, secs):
        reps = 0
        t0 = time.perf_counter()
        while True:
            qa = oracle.quantize(np.ascontiguousarray(A_bits[:r]), oracle.MXFP4)
            qb = oracle.quantize(np.ascontiguousarray(B_bits[:nb]), oracle.MXFP4)
            Ad = oracle.dequantize_f64(oracle.MXFP4, qa[0], qa[1], r, K)
            Bd = oracle.dequantize_f64(oracle.MXFP4, qb[0], qb[1], nb, K)
            oracle.gemm(Ad, Bd)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= secs:
                return reps, dt

    reps, dt = run(rows, N, min_seconds)
    # the same on one thread, on a sixteenth of the output (rows / 16 x N / ... )
    oracle.set_threads(1)
    r1 = max(rows // 16, 1)
    reps1, dt1 = run(r1, N, min_seconds / 2)
    oracle.set_threads(threads)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": 2.0 * rows * N * K * reps / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": dt, "cpu_model": cpu, "cpus_visible": os.cpu_count(),
            "one_thread_value": 2.0 * r1 * N * K * reps1 / dt1 / 1e12, "one_thread_seconds": dt1,
            "sample": f"{reps} repetitions of: MXFP4 quantize of {rows} rows of A and all {N} rows "
                      f"of B, then {rows} of the {M} output rows of the FP64 GEMM (K={K}); "
                      f"throughput = {reps}*2*{rows}*{N}*{K} / time; one thread: {reps1} repetitions "
                      f"with {r1} rows of A"}


def device_facts(torch):
    """The box's own figures: compute units and clock from the device
    properties (peaks derived from them: dense FP4/FP6 16384, FP8 8192, BF16
    4096 flop per clock and CU), and a device-to-device copy of 1 GiB as the
    practical HBM ceiling (read + write bytes / time)."""
    p = torch.cuda.get_device_properties(0)
    cus = int(p.multi_processor_count)
    clk = None
    try:
        from ctypes import CDLL, byref, c_int
        hip = CDLL("libamdhip64.so")
        v = c_int(0)
        if hip.hipDeviceGetAttribute(byref(v), 5, 0) == 0:  # hipDeviceAttributeClockRate (kHz)
            clk = v.value / 1e6
    except OSError:
        pass
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = time_fn(torch, lambda: dst.copy_(src), 10, 3)
    del src, dst
    out = {"compute_units": cus, "max_clock_ghz": clk, "copy_gbs_1gib": 2 * (1 << 30) / ms / 1e6,
           "copy_frac_of_8tbs": 2 * (1 << 30) / ms / 1e6 / PEAK_HBM_GBS}
    if clk:
        out["peak_tflops_from_clock"] = {k: cus * f * clk * 1e9 / 1e12 for k, f in
                                         (("fp4", 16384), ("fp8", 8192), ("bf16", 4096))}
    return out


def detail(torch, mx, W, args):
    """Secondary workloads (each timed in isolation, median over iterations)."""
    res = {}
    it, wu = 20, 5
    g = torch.Generator(device="cuda")
    g.manual_seed(0)

    def randn(r, c, std=1.0):
        return (torch.randn(r, c, generator=g, device="cuda", dtype=torch.float32) * std).to(torch.bfloat16)

    # MXFP8 4096^3 GEMM: exact (FP8 converted to BF16) and the native FP8 instruction
    M = N = K = 4096
    a, b = randn(M, K), randn(N, K, 0.02)
    qa, qb = mx.empty(1, M, K), mx.empty(1, N, K)
    mx.mx_quantize(a, qa)
    mx.mx_quantize(b, qb)
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ms = time_fn(torch, lambda: mx.mx_gemm(qa, qb, C), it, wu)
    res["mxfp8_gemm_4096_exact"] = {"ms": ms, "tflops": 2 * M * N * K / ms / 1e9,
                                    "frac_fp8_peak": 2 * M * N * K / ms / 1e9 / PEAK_TFLOPS["fp8"],
                                    "frac_bf16_peak": 2 * M * N * K / ms / 1e9 / PEAK_TFLOPS["bf16"]}
    ms = time_fn(torch, lambda: mx.mx_gemm_ex(qa, qb, C, mx.MX_GEMM_FP8_NATIVE), it, wu)
    res["mxfp8_gemm_4096_native_fp8"] = {"ms": ms, "tflops": 2 * M * N * K / ms / 1e9,
                                         "frac_fp8_peak": 2 * M * N * K / ms / 1e9 / PEAK_TFLOPS["fp8"]}
    qat, qbt = mx.empty(1, M, K, layout=mx.MX_LAYOUT_TILED), mx.empty(1, N, K, layout=mx.MX_LAYOUT_TILED)
    mx.mx_quantize(a, qat)
    mx.mx_quantize(b, qbt)
    ms = time_fn(torch, lambda: mx.mx_gemm_ex(qat, qbt, C, mx.MX_GEMM_FP8_NATIVE), it, wu)
    res["mxfp8_gemm_4096_native_fp8_tiled"] = {"ms": ms, "tflops": 2 * M * N * K / ms / 1e9,
                                               "frac_fp8_peak": 2 * M * N * K / ms / 1e9 / PEAK_TFLOPS["fp8"]}
    mx.mx_quantize(a, qa)
    ms = time_fn(torch, lambda: mx.mx_quantize(a, qa), it, wu)
    by = M * K * (2 + 1 + 1 / 32)
    res["mxfp8_quantize_4096x4096"] = {"ms": ms, "gbs": by / ms / 1e6, "frac_hbm": by / ms / 1e6 / PEAK_HBM_GBS}
    # NVFP4 4096^3 (E4M3 block scales applied explicitly, FP16 instruction)
    qna, qnb = mx.empty(3, M, K), mx.empty(3, N, K)
    mx.mx_quantize(a, qna, amax=torch.zeros(1, device="cuda"))
    mx.mx_quantize(b, qnb, amax=torch.zeros(1, device="cuda"))
    ms = time_fn(torch, lambda: mx.mx_gemm(qna, qnb, C), it, wu)
    res["nvfp4_gemm_4096"] = {"ms": ms, "tflops": 2 * M * N * K / ms / 1e9,
                              "kernel": "k_gemm_nv_pipe (E2M1 x E4M3 to exact FP16, FP16 instruction)",
                              "frac_fp4_peak": 2 * M * N * K / ms / 1e9 / PEAK_TFLOPS["fp4"],
                              "frac_bf16_peak": 2 * M * N * K / ms / 1e9 / PEAK_TFLOPS["bf16"]}
    del qna, qnb
    # MXFP4 4096^3 on row-major operands (LDS-pipelined kernel), for comparison
    q4a, q4b = mx.empty(2, M, K), mx.empty(2, N, K)
    mx.mx_quantize(a, q4a)
    mx.mx_quantize(b, q4b)
    ms = time_fn(torch, lambda: mx.mx_gemm(q4a, q4b, C), it, wu)
    res["mxfp4_gemm_4096_rows_layout"] = {"ms": ms, "tflops": 2 * M * N * K / ms / 1e9,
                                          "frac_fp4_peak": 2 * M * N * K / ms / 1e9 / PEAK_TFLOPS["fp4"]}
    # fused quantize-and-GEMM: the 4096^3 MXFP4 product written as MXFP4 (tile layout) by the
    # GEMM's epilogue, against the product written in BF16 and quantized by a second kernel
    q4at, q4bt = mx.empty(2, M, K, layout=mx.MX_LAYOUT_TILED), mx.empty(2, N, K, layout=mx.MX_LAYOUT_TILED)
    mx.mx_quantize(a, q4at)
    mx.mx_quantize(b, q4bt)
    q4c = mx.empty(2, M, N, layout=mx.MX_LAYOUT_TILED)
    ms_fr = time_fn(torch, lambda: mx.mx_gemm_quantize(q4at, q4bt, q4c), it, wu)
    ms_fs = time_fn(torch, lambda: mx.mx_gemm_quantize(q4at, q4bt, q4c, mx.MX_SR, 1, 0), it, wu)

    def two_step(rnd):
        mx.mx_gemm(q4at, q4bt, C)
        mx.mx_quantize(C, q4c, rnd, 1, 0)
    ms_tr = time_fn(torch, lambda: two_step(mx.MX_RNE), it, wu)
    ms_ts = time_fn(torch, lambda: two_step(mx.MX_SR), it, wu)
    # the same product written as MXFP8 E5M2 with SR (a gradient's format), tile layout
    q5c = mx.empty(mx.MX_MXFP8_E5M2, M, N, layout=mx.MX_LAYOUT_TILED)
    ms_f5 = time_fn(torch, lambda: mx.mx_gemm_quantize(q4at, q4bt, q5c, mx.MX_SR, 1, 0), it, wu)
    res["mxfp4_gemm_quantize_4096_fused_e5m2_sr"] = {"ms": ms_f5, "tflops": 2 * M * N * K / ms_f5 / 1e9,
                                                     "kernel": "k_gemm_mx_tiled_q<MXFP4, E5M2, SR, tiled>"}
    del q5c
    res["mxfp4_gemm_quantize_4096_fused"] = {
        "fused_rne_ms": ms_fr, "fused_rne_tflops": 2 * M * N * K / ms_fr / 1e9, "two_step_rne_ms": ms_tr,
        "fused_sr_ms": ms_fs, "two_step_sr_ms": ms_ts}
    del q4at, q4bt, q4c
    # fused quantize-and-GEMM, prologue half: A arrives in BF16 and is quantized inside the
    # GEMM (Q(A) also written out), against mx_quantize followed by mx_gemm
    qa_out = mx.empty(1, M, K)
    ms_q8 = time_fn(torch, lambda: mx.mx_gemm_quantize_a(a, mx.MX_MXFP8_E4M3, qb, C, a_out=qa_out), it, wu)

    def two_step_a8():
        mx.mx_quantize(a, qa)
        mx.mx_gemm(qa, qb, C)
    ms_t8 = time_fn(torch, two_step_a8, it, wu)
    q4o = mx.empty(2, M, K)
    ms_q4 = time_fn(torch, lambda: mx.mx_gemm_quantize_a(a, mx.MX_MXFP4_E2M1, q4b, C, a_out=q4o), it, wu)

    def two_step_a4():
        mx.mx_quantize(a, q4a)
        mx.mx_gemm(q4a, q4b, C)
    ms_t4 = time_fn(torch, two_step_a4, it, wu)
    res["gemm_4096_quantize_a_in_prologue"] = {
        "mxfp8_fused_ms": ms_q8, "mxfp8_fused_tflops": 2 * M * N * K / ms_q8 / 1e9,
        "mxfp8_two_step_ms": ms_t8, "mxfp4_fused_ms": ms_q4, "mxfp4_fused_tflops": 2 * M * N * K / ms_q4 / 1e9,
        "mxfp4_two_step_rows_layout_ms": ms_t4,
        "kernel": "k_gemm_qa (A quantized per 32-element block in registers, decoded to exact BF16 in LDS, "
                  "BF16 instruction); two-step: mx_quantize then the exact MXFP8 / row-layout MXFP4 GEMM"}
    del qa_out, q4o
    # MXFP4 tile-layout quantize of the activation operand, floor and ceil scale rules
    q4t = mx.empty(2, M, K, layout=mx.MX_LAYOUT_TILED)
    by4 = M * K * (2 + 0.5 + 1 / 32)
    for name, fl_ in (("floor", 0), ("ceil", mx.MX_FLAG_SCALE_CEIL)):
        ms = time_fn(torch, lambda: mx.mx_quantize(a, q4t, flags=fl_), it, wu)
        res[f"mxfp4_quantize_tiled_4096x4096_{name}"] = {"ms": ms, "gbs": by4 / ms / 1e6,
                                                         "frac_hbm": by4 / ms / 1e6 / PEAK_HBM_GBS}
    del q4t
    del a, b, qa, qb, qat, qbt, q4a, q4b, C

    # NVFP4 MoE forward: 4096 tokens x 7168, top-8 of 32 experts, W_e 2048x7168
    tokens, hid, E, topk, inter = 4096, 7168, 32, 8, 2048
    X = randn(tokens, hid)
    row_index, offsets = W.uniform_topk_routing(tokens, E, topk, 0, 6)
    R = int(offsets[-1])
    Wt = randn(E * inter, hid, 0.02)
    qw = mx.empty(3, E * inter, hid, n_tensor_scales=E)
    amax = torch.zeros(E, dtype=torch.float32, device="cuda")
    for e in range(E):
        mx.mx_quantize(Wt[e * inter:(e + 1) * inter], qw.view_rows(e * inter, (e + 1) * inter, qw.tensor_scale[e:e + 1]),
                       amax=amax[e:e + 1])
    # the same expert weights with 2-D 16x16 blocks (each expert: amax pass + encode pass)
    qw2 = mx.empty(3, E * inter, hid, n_tensor_scales=E)

    def quant_experts_2d():
        for e in range(E):
            mx.mx_quantize(Wt[e * inter:(e + 1) * inter],
                           qw2.view_rows(e * inter, (e + 1) * inter, qw2.tensor_scale[e:e + 1]),
                           flags=mx.MX_FLAG_BLOCK_2D, amax=amax[e:e + 1])
    ms_w2_calls = time_fn(torch, quant_experts_2d, 5, 2)
    # the same 32 quantizations as one mx_quantize_batch call (NVFP4 jobs share
    # the amax and encode launches, 16 per launch)
    batch_2d = mx.QuantizeBatch([dict(x=Wt[e * inter:(e + 1) * inter],
                                      out=qw2.view_rows(e * inter, (e + 1) * inter, qw2.tensor_scale[e:e + 1]),
                                      flags=mx.MX_FLAG_BLOCK_2D, amax=amax[e:e + 1]) for e in range(E)])
    ms_w2 = time_fn(torch, batch_2d.run, 5, 2)
    byw = E * inter * hid * (2 * 2 + 0.5 + 1 / 16)
    res["nvfp4_2d_weights_32x2048x7168"] = {"ms_all_experts": ms_w2, "ms_one_call_per_expert": ms_w2_calls,
                                            "call": "mx_quantize_batch (32 jobs)",
                                            "gbs_2pass": byw / ms_w2 / 1e6,
                                            "frac_hbm": byw / ms_w2 / 1e6 / PEAK_HBM_GBS}
    del Wt, qw2
    qx = mx.empty(3, tokens, hid)
    xa = torch.zeros(1, dtype=torch.float32, device="cuda")
    ri = torch.from_numpy(row_index).cuda()
    off = torch.from_numpy(offsets).cuda()
    Cg = torch.empty(R, inter, dtype=torch.bfloat16, device="cuda")
    ms_q = time_fn(torch, lambda: mx.mx_quantize(X, qx, amax=xa), it, wu)
    ms_q46 = time_fn(torch, lambda: mx.mx_quantize(X, qx, flags=mx.MX_FLAG_FOUR_OVER_SIX, amax=xa), it, wu)
    ms_g = time_fn(torch, lambda: mx.mx_gemm_grouped(qx, ri, R, qw, E, off, Cg), it, wu)
    fl = 2.0 * R * inter * hid
    by = tokens * hid * (2 * 2 + 0.5 + 1 / 16)
    res["nvfp4_moe_fwd"] = {"quant_ms": ms_q, "quant_gbs_2pass": by / ms_q / 1e6,
                            "quant_four_over_six_ms": ms_q46,
                            "quant_four_over_six_gbs_2pass": by / ms_q46 / 1e6,
                            "gemm_ms": ms_g, "gemm_tflops": fl / ms_g / 1e9,
                            "frac_fp4_peak": fl / ms_g / 1e9 / PEAK_TFLOPS["fp4"],
                            "frac_fp8_peak": fl / ms_g / 1e9 / PEAK_TFLOPS["fp8"],
                            "frac_bf16_peak": fl / ms_g / 1e9 / PEAK_TFLOPS["bf16"]}
    del X, qw, qx, Cg

    # backward: NVFP4 X [16384, 4096] -> MXFP8 X^T (SR); dY [16384, 14336] -> MXFP8 dY^T (SR);
    # wgrad GEMM M=4096 N=14336 K=16384 -> FP32
    T_, H, O = 16384, 4096, 14336
    Xb = randn(T_, H)
    qx = mx.empty(3, T_, H)
    mx.mx_quantize(Xb, qx, amax=torch.zeros(1, device="cuda"))
    xt = mx.empty(1, H, T_)
    ms_r = time_fn(torch, lambda: mx.mx_requant_transpose(xt, src=qx, rnd=mx.MX_SR, seed=0, counter=0), it, wu)
    by_r = T_ * H * (0.5 + 1 / 16 + 1 + 1 / 32)
    del Xb
    dY = randn(T_, O)
    dyt = mx.empty(1, O, T_)
    ms_d = time_fn(torch, lambda: mx.mx_requant_transpose(dyt, x_bf16=dY, rnd=mx.MX_SR, seed=0, counter=T_ * H // 8), it, wu)
    by_d = T_ * O * (2 + 1 + 1 / 32)
    del dY
    Cw = torch.empty(H, O, dtype=torch.float32, device="cuda")
    ms_w = time_fn(torch, lambda: mx.mx_gemm(xt, dyt, Cw), 5, 2)
    ms_wn = time_fn(torch, lambda: mx.mx_gemm_ex(xt, dyt, Cw, mx.MX_GEMM_FP8_NATIVE), 5, 2)
    fl = 2.0 * H * O * T_
    res["backward_requant_wgrad"] = {
        "requant_nvfp4_ms": ms_r, "requant_gbs": by_r / ms_r / 1e6, "requant_frac_hbm": by_r / ms_r / 1e6 / PEAK_HBM_GBS,
        "dy_quant_t_ms": ms_d, "dy_gbs": by_d / ms_d / 1e6, "dy_frac_hbm": by_d / ms_d / 1e6 / PEAK_HBM_GBS,
        "wgrad_exact_ms": ms_w, "wgrad_exact_tflops": fl / ms_w / 1e9,
        "wgrad_native_fp8_ms": ms_wn, "wgrad_native_fp8_tflops": fl / ms_wn / 1e9}
    del qx, xt, dyt, Cw

    # S2F6 combine codec on the MoE combine tensor (32768 routed rows x 7168, BF16): encode
    # = Hadamard transform + block-scaled INT8 (RNE), decode = INT8 + inverse transform to BF16
    Rc, Hc = 32768, 7168
    Xc = randn(Rc, Hc)
    qc = mx.empty(mx.MX_MXINT8, Rc, Hc)
    Yc = torch.empty(Rc, Hc, dtype=torch.bfloat16, device="cuda")
    mask_c = mx.mx_rht_signs(0)
    ms_e = time_fn(torch, lambda: mx.mx_quantize(Xc, qc, flags=mx.MX_FLAG_RHT16, sign_mask=mask_c), it, wu)
    ms_d = time_fn(torch, lambda: mx.mx_dequantize(qc, Yc, mx.MX_FLAG_RHT16, mask_c), it, wu)
    by_e = Rc * Hc * (2 + 1 + 1 / 32)
    res["s2f6_combine_codec_32768x7168"] = {
        "encode_ms": ms_e, "encode_gbs": by_e / ms_e / 1e6, "encode_frac_hbm": by_e / ms_e / 1e6 / PEAK_HBM_GBS,
        "decode_ms": ms_d, "decode_gbs": by_e / ms_d / 1e6, "decode_frac_hbm": by_e / ms_d / 1e6 / PEAK_HBM_GBS,
        "bits_per_value": 8.25}
    # the other element types: quantize 8192x7168 BF16 (RNE)
    Xq = Xc[:8192]
    for name, f in (("mxint8", mx.MX_MXINT8), ("mxfp8_e5m2", mx.MX_MXFP8_E5M2),
                    ("mxfp6_e3m2", mx.MX_MXFP6_E3M2), ("mxfp6_e2m3", mx.MX_MXFP6_E2M3)):
        qf = mx.empty(f, 8192, Hc)
        ms_f = time_fn(torch, lambda: mx.mx_quantize(Xq, qf), it, wu)
        byf = 8192 * Hc * (2 + (0.75 if "fp6" in name else 1) + 1 / 32)
        res[f"{name}_quantize_8192x7168"] = {"ms": ms_f, "gbs": byf / ms_f / 1e6,
                                             "frac_hbm": byf / ms_f / 1e6 / PEAK_HBM_GBS}
        del qf
    del Xc, qc, Yc, Xq
    # products of the other MX formats and mixed pairs (4096^3, BF16 out)
    M2 = 4096
    Xa, Xb = randn(M2, M2), randn(M2, M2, 0.02)
    Cm = torch.empty(M2, M2, dtype=torch.bfloat16, device="cuda")
    # (FP6 pairs other than E3M2 x E3M2 run on the scaled FP6/FP4 instruction,
    # k_gemm_mx_f6; FP8 pairs with E5M2 and MXINT8 x MXINT8 on the exact 8-bit
    # pipeline; the rest decode to BF16 in k_gemm_mx_any)
    for name, fa_, fb_, native in (("mxint8_x_mxint8", mx.MX_MXINT8, mx.MX_MXINT8, None),
                                   ("e5m2_x_e4m3", mx.MX_MXFP8_E5M2, mx.MX_MXFP8_E4M3, None),
                                   ("fp6_e3m2_x_fp6_e3m2", mx.MX_MXFP6_E3M2, mx.MX_MXFP6_E3M2, "bf16"),
                                   ("fp6_e2m3_x_fp6_e2m3", mx.MX_MXFP6_E2M3, mx.MX_MXFP6_E2M3, True),
                                   ("fp6_e2m3_x_fp4", mx.MX_MXFP6_E2M3, mx.MX_MXFP4_E2M1, True),
                                   ("fp6_e3m2_x_fp4", mx.MX_MXFP6_E3M2, mx.MX_MXFP4_E2M1, True)):
        qa_, qb_ = mx.empty(fa_, M2, M2), mx.empty(fb_, M2, M2)
        mx.mx_quantize(Xa, qa_)
        mx.mx_quantize(Xb, qb_)
        ms_m = time_fn(torch, lambda: mx.mx_gemm(qa_, qb_, Cm), it, wu)
        tf = 2 * M2**3 / ms_m / 1e9
        res[f"gemm_4096_{name}"] = {"ms": ms_m, "tflops": tf,
                                    "kernel": {True: "k_gemm_mx_f6 (scaled FP6/FP4 instruction)",
                                               None: "k_gemm_mx8_exact (8-bit codes converted to BF16 after the "
                                                     "fragment reads)",
                                               "bf16": "k_gemm_mx_f6<E3M2, E3M2> (decoded to BF16 in the FP6 kernel) "
                                                       "+ k_gemm_mx_any fix-up scan",
                                               False: "k_gemm_mx_any (exact BF16 decode)"}[native],
                                    "frac_peak": tf / PEAK_TFLOPS["fp6" if native is True else "bf16"],
                                    "peak": "fp6" if native is True else "bf16"}
        del qa_, qb_
    # E5M2 x E4M3 in the row layout on the scaled FP8 instruction (MX_GEMM_FP8_NATIVE)
    qa_, qb_ = mx.empty(mx.MX_MXFP8_E5M2, M2, M2), mx.empty(mx.MX_MXFP8_E4M3, M2, M2)
    mx.mx_quantize(Xa, qa_)
    mx.mx_quantize(Xb, qb_)
    ms_m = time_fn(torch, lambda: mx.mx_gemm_ex(qa_, qb_, Cm, mx.MX_GEMM_FP8_NATIVE), it, wu)
    res["gemm_4096_e5m2_x_e4m3_native_fp8_rows"] = {"ms": ms_m, "tflops": 2 * M2**3 / ms_m / 1e9,
                                                    "frac_fp8_peak": 2 * M2**3 / ms_m / 1e9 / PEAK_TFLOPS["fp8"],
                                                    "kernel": "k_gemm_mx_pipe<MXFP8, BF16, E5M2, E4M3>"}
    del qa_, qb_
    # E5M2 x E4M3 in the tile layout on the scaled FP8 instruction (MX_GEMM_FP8_NATIVE)
    qa_ = mx.empty(mx.MX_MXFP8_E5M2, M2, M2, layout=mx.MX_LAYOUT_TILED)
    qb_ = mx.empty(mx.MX_MXFP8_E4M3, M2, M2, layout=mx.MX_LAYOUT_TILED)
    mx.mx_quantize(Xa, qa_)
    mx.mx_quantize(Xb, qb_)
    ms_m = time_fn(torch, lambda: mx.mx_gemm_ex(qa_, qb_, Cm, mx.MX_GEMM_FP8_NATIVE), it, wu)
    res["gemm_4096_e5m2_x_e4m3_native_fp8_tiled"] = {"ms": ms_m, "tflops": 2 * M2**3 / ms_m / 1e9,
                                                     "frac_fp8_peak": 2 * M2**3 / ms_m / 1e9 / PEAK_TFLOPS["fp8"]}
    del qa_, qb_, Xa, Xb, Cm

    # RHT16 + NVFP4 SR of an 8192x7168 Student-t(3) gradient (two passes)
    G = torch.distributions.StudentT(3.0).sample((8192, 7168)).to(device="cuda", dtype=torch.bfloat16)
    qg = mx.empty(3, 8192, 7168)
    ga = torch.zeros(1, device="cuda")
    mask = mx.mx_rht_signs(0)
    ms_h = time_fn(torch, lambda: mx.mx_quantize(G, qg, mx.MX_SR, 0, 0, mx.MX_FLAG_RHT16, mask, ga), it, wu)
    by2 = 8192 * 7168 * (2 * 2 + 0.5 + 1 / 16)
    res["rht_nvfp4_sr_8192x7168"] = {"ms": ms_h, "gbs_2pass": by2 / ms_h / 1e6,
                                     "frac_hbm": by2 / ms_h / 1e6 / PEAK_HBM_GBS}
    # round-trip error statistics of the same tensor: quantize, decode (inverse
    # transform where the forward one was used), compare -- all on the device
    Y = torch.empty(8192, 7168, dtype=torch.float32, device="cuda")
    st = torch.empty(4, dtype=torch.float64, device="cuda")
    rt = {}
    n = 8192 * 7168
    for rnd_name, rnd in (("rne", mx.MX_RNE), ("sr", mx.MX_SR)):
        for rht in (False, True):
            fl_ = mx.MX_FLAG_RHT16 if rht else 0
            mx.mx_quantize(G, qg, rnd, 0, 0, fl_, mask, ga)
            ms_dq = time_fn(torch, lambda: mx.mx_dequantize(qg, Y, fl_, mask), it, wu)
            ms_st = time_fn(torch, lambda: mx.mx_error_stats(G, Y, st), it, wu)
            v = st.cpu().numpy()
            rt[f"{rnd_name}_{'rht' if rht else 'plain'}"] = {
                "rel_rmse": float(np.sqrt(v[0] / v[1])), "mean_err": float(v[2] / n),
                "max_abs_err": float(v[3]), "dequant_ms": ms_dq, "stats_ms": ms_st}
    rt["source"] = "Student-t(3) 8192x7168 BF16 (torch sampler), NVFP4 E2M1/E4M3/16 + FP32 tensor scale"
    res["nvfp4_roundtrip_stats_8192x7168"] = rt
    del G, qg, Y
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the path is built and measured on one MI355X "
              "(sharding across GPUs is not built); --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)
    import microscaling_precision_gemm_amd as mx
    import workloads as W
    mx.load()
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    dev = device_facts(torch)
    h = headline(torch, mx, W, args)
    roof = {"bound": "mfma", "achieved": h["gemm_tflops"], "peak": PEAK_TFLOPS["fp4"],
            "unit": "TFLOP/s", "frac": h["gemm_tflops"] / PEAK_TFLOPS["fp4"], "traffic": gemm_traffic(),
            "traffic_unit": "bytes per launch", "algorithmic_bytes": 2 * 4096 * 4096 * (0.5 + 1 / 32) + 4096 * 4096 * 2,
            "kernel": "k_gemm_mx_tiled<MXFP4, BF16 out> (256x256 per workgroup, tile layout)",
            "gemm_ms": h["gemm_ms"],
            "gemm_ms_how": "median over 5 pairs of (batch of steps - batch of the quantize launches alone), "
                           "HIP events on the launch stream",
            "gemm_ms_back_to_back": h["gemm_ms_back_to_back"]}
    line = {
        "metric": "block-scaled GEMM TFLOPS (MXFP4/NVFP4/MXFP8 4096^3) + quantize HBM GB/s",
        "value": h["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "MXFP4 E2M1 quantize (RNE, E8M0/32) of A 4096x4096 BF16 N(0,1) "
                               "with 1% of K-columns x50 and B 4096x4096 BF16 N(0,0.02^2), then "
                               "block-scaled GEMM M=N=K=4096, FP32 accumulate, BF16 out",
                   "M": 4096, "N": 4096, "K": 4096, "input_rotation": 16, "launch": h["launch"],
                   "layout": "mx tile layout"},
        "roofline": roof,
        "device": dev,
        "quantize": {"ms_per_operand": h["quant_ms"], "achieved_gbs": h["quant_gbs"],
                     "peak_gbs": PEAK_HBM_GBS, "frac": h["quant_gbs"] / PEAK_HBM_GBS,
                     "bytes_per_operand": h["qbytes"],
                     "kernel": "k_quant_mx_tiled_batch<BF16, MXFP4, RNE> (A and B in one launch; "
                               "time per launch / 2)"},
    }
    if not args.no_cpu_baseline:
        import oracle
        line["cpu_baseline"] = cpu_baseline(W, oracle, h["A_bits"], h["B_bits"], args.cpu_rows)
    if not args.no_detail:
        line["detail"] = detail(torch, mx, W, args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
