"""Benchmark of the static per-tensor FP8 linear layer on one MI355X.

One step = the shared-QKV projection group in W8A8 mode at its full size:
x bf16 [16384, 4096] is quantized once to E4M3 with its static input scale
(fp8lin_quantize_static), then the three E4M3 4096 -> 4096 projections with
distinct weight scales run on it in one grouped launch
(fp8lin_gemm_w8a8_group, HIP events around it). `value` is the GEMM work of
the step, 3 x 2 M N K, over the step's wall time (quantization included),
in TFLOP/s.

In the same run, on the same resident inputs:
  * w8a16     the 16-bit step of the same projections (fp8lin_qkv_shared in
              W8A16 mode: one grouped launch, no quantization)
  * rows      every other hot-path call at its workload size: the same step
              as three separate fp8lin_gemm_w8a8 calls, fp8lin_qkv_shared in
              both modes, quantize and SwiGLU (GB/s,
              input/output buffers rotated over > 512 MB so the 256 MB
              last-level cache cannot serve repeats), the gated-MLP GEMMs,
              the gate/up + SwiGLU step split and fused,
              the 1024- and 8192-row projections, the dynamic-FP8 form of the
              step, the per-head QK RMSNorm + RoPE on the step's Q and K, the
              binary16 / float32 activation forms of W8A16 and SwiGLU, the
              step policy, and the 8-step denoising schedule over 4 blocks
              (config 5)
  * roofline  the grouped W8A8 GEMM launch against the dense FP8 matrix-core
              peak
  * cpu_baseline  the CPU oracle on a bounded sample of the same step

Usage: python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
       (defaults K = W = 100; after the W warm-up steps, further untimed
       steps run for about 30 ms of device time, reported as settle_ms: the
       matrix cores reach their sustained clock only after some tens of
       milliseconds of load, and every row gets the same settling)
       python bench.py --pmc   (a few launches of each step kernel and a
                                plain copy, for rocprofv3 counter runs)
       python bench.py --schedule-only   (the 8-step schedule row alone,
                                for its kernel trace)
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import w8a16_linear_layers_amd as fp8lin  # noqa: E402
from workloads import config2, config3, config4, norm_weight_bf16, normal_bf16, rope_tables  # noqa: E402

METRIC = "W8A8 FP8 GEMM TFLOP/s (% FP8 MFMA peak) at M=16384,K=N=4096; W8A16 TFLOP/s"
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 matrix-core peak
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 matrix-core peak
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
M, K, N = 16384, 4096, 4096
GEMM_FLOP = 2.0 * M * N * K
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w8a8_group3_16384x4096x4096_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "w8a16_linear_layers_amd", "csrc", "gemm.hip")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def timed(fn, reps, warmup=3, warm_ms=30.0):
    """Average device time of fn() over `reps` calls (HIP events on the current stream), ms.

    Before timing, fn() runs for about `warm_ms` of device time (sized from one timed call): the shader
    clock takes a few tens of milliseconds to settle under matrix-core load, and short rows timed right
    after a different shape would otherwise read low."""
    for _ in range(warmup):
        fn()
    e0, e1 = events(2)
    torch.cuda.synchronize()
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(min(2000, int(warm_ms / max(e0.elapsed_time(e1), 1e-3)))):
        fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def timed_graph(fn, reps, calls=20, warm_ms=30.0):
    """Average device time per fn() call, ms, with `calls` calls captured in one HIP graph and the graph
    replayed `reps` times: the kernels then run back to back, without the host's per-call launch time
    between them (what a serving loop that replays a captured step sees). fn() must write only buffers
    allocated before capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture stream
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    settle(graph.replay, warm_ms)
    e0, e1 = events(2)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * calls)


def settle(fn, warm_ms=30.0):
    """Run fn() for about `warm_ms` of device time (sized from one timed call), so that the shader clock
    has settled under the load before timing starts; returns the device time spent, ms."""
    e0, e1 = events(2)
    torch.cuda.synchronize()
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    n = min(2000, int(np.ceil(warm_ms / max(e0.elapsed_time(e1), 1e-3))))
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def rotating(make, total_bytes, per_set_bytes):
    sets = max(2, int(np.ceil(total_bytes / per_set_bytes)))
    return [make(i) for i in range(sets)]


def gemm_traffic():
    """HBM bytes per grouped GEMM launch from the committed rocprofv3 counter runs, if current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    with open(GEMM_SOURCE, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if rec.get("gemm_source_sha256") != digest:
        return None  # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


def cpu_baseline(case, rows=16384, cols=4096):
    """The oracle's W8A8 step on a bounded sample: `rows` rows x `cols` output columns per projection."""
    from threadpoolctl import threadpool_info

    from oracle import linear

    x = case.x[:rows].float().numpy()
    qws = [linear.quantize_static(w[:cols].float().numpy(), s) for w, s in zip(case.ws, case.weight_scales)]
    t0 = time.perf_counter()
    q = linear.quantize_static(x, case.input_scale)
    for qw, s in zip(qws, case.weight_scales):
        linear.gemm_w8a8(q, qw, case.input_scale, s)
    dt = time.perf_counter() - t0
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    flop = 3 * 2.0 * rows * cols * K
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d rows x first %d output columns of each of the 3 projections (activation quantization + "
        "3 float64 W8A8 GEMMs), %.1f s" % (rows, cols, dt),
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


def pmc_mode(dev):
    """A few launches of each kernel plus a plain copy of known size, for counter runs."""
    case = config3()
    x = case.x.to(dev)
    qws = [fp8lin.fp8lin_quantize_static(w.to(dev), s) for w, s in zip(case.ws, case.weight_scales)]
    qx = fp8lin.fp8lin_quantize_static(x, case.input_scale)
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    src = torch.ones(256 * 2**20, dtype=torch.uint8, device=dev)  # 256 MiB plain copy
    dst = torch.empty_like(src)
    sw = case.weight_scales
    # the SwiGLU at [8192, 16384] (E4M3 and bf16 out) and the QK RMSNorm + RoPE on Q and K [16384, 4096]
    mi, inter, hd = 8192, 16384, 128
    g = normal_bf16((mi, inter), 0.45, 910).to(dev)
    u = normal_bf16((mi, inter), 0.45, 911).to(dev)
    h8 = torch.empty((mi, inter), dtype=torch.uint8, device=dev)
    h16 = torch.empty((mi, inter), dtype=torch.bfloat16, device=dev)
    cq, sq = (v.to(dev) for v in rope_tables(M, hd))
    wq, wk = norm_weight_bf16(hd, 950).to(dev), norm_weight_bf16(hd, 951).to(dev)
    qo, ko = torch.empty_like(ys[0]), torch.empty_like(ys[1])
    for _ in range(3):
        dst.copy_(src)
        fp8lin.fp8lin_quantize_static(x, case.input_scale, out=qx)
        fp8lin.fp8lin_gemm_w8a8_group(qx, qws, case.input_scale, sw, outs=ys)
        fp8lin.fp8lin_qkv_shared(x, qws, sw, [case.input_scale] * 3, fp8lin.MODE_W8A16, outs=ys)
        fp8lin.fp8lin_swiglu_2in_quant(g, u, 2.1 / 448, fp8lin.DT_E4M3, out=h8)
        fp8lin.fp8lin_swiglu_2in_quant(g, u, 1.0, fp8lin.DT_BF16, out=h16)
        fp8lin.fp8lin_qk_norm_rope(ys[0], ys[1], wq, wk, cq, sq, hd, 1e-6, q_out=qo, k_out=ko)
    torch.cuda.synchronize()
    log("pmc mode done: 3 x (copy 256 MiB, quantize, grouped gemm_w8a8, grouped gemm_w8a16 (3 projections of "
        "16384x4096x4096), swiglu 8192x16384 E4M3 out, swiglu bf16 out, qk_norm_rope 16384 x 2 x 32 heads of 128)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--no-schedule", action="store_true", help="skip the 8-step schedule row")
    ap.add_argument("--pmc", action="store_true")
    ap.add_argument("--schedule-only", action="store_true",
                    help="only the 8-step schedule row (one warm-up and two timed schedules), for kernel traces")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(
            "bench.py measures one MI355X: the static-FP8 linear layer is benchmarked on a single GPU, with no "
            "cross-GPU exchange (--gpus %d, WORLD_SIZE %d requested). Run with --gpus 1." % (args.gpus, world),
            file=sys.stderr,
        )
        sys.exit(2)
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    fp8lin.load_library()
    dev = torch.device("cuda", 0)
    if args.pmc:
        pmc_mode(dev)
        return
    if args.schedule_only:
        print(json.dumps({"schedule_cfg5": schedule_cfg5(dev, step_policy_of_workload())}), flush=True)
        return

    log("generating the shared-QKV workload (x [16384, 4096], three 4096x4096 weights)")
    case = config3()
    x = case.x.to(dev)
    s_in = case.input_scale
    qws = [fp8lin.fp8lin_quantize_static(w.to(dev), s) for w, s in zip(case.ws, case.weight_scales)]
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    stream = torch.cuda.current_stream()

    def step_w8a8(ev=None):
        fp8lin.fp8lin_quantize_static(x, s_in, out=qx)
        if ev is not None:
            ev[0].record(stream)
        fp8lin.fp8lin_gemm_w8a8_group(qx, qws, s_in, case.weight_scales, outs=ys)
        if ev is not None:
            ev[1].record(stream)

    def step_w8a16():
        fp8lin.fp8lin_qkv_shared(x, qws, case.weight_scales, [s_in] * 3, fp8lin.MODE_W8A16, outs=ys)

    for _ in range(args.warmup):
        step_w8a8()
    settle_ms = settle(step_w8a8)
    log("timing %d W8A8 steps" % args.steps)
    gemm_ev = [events(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step_w8a8(gemm_ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gemm_ms = [ev[0].elapsed_time(ev[1]) for ev in gemm_ev]
    gemm_avg_ms = float(np.mean(gemm_ms))
    value = 3 * GEMM_FLOP / (ms_per_step * 1e-3) / 1e12

    for _ in range(args.warmup):
        step_w8a16()
    settle16_ms = settle(step_w8a16)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_w8a16()
    torch.cuda.synchronize()
    ms16 = (time.perf_counter() - t0) * 1e3 / args.steps
    tf16 = 3 * GEMM_FLOP / (ms16 * 1e-3) / 1e12

    achieved = 3 * GEMM_FLOP / (gemm_avg_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        # after the warm-up steps, further untimed steps for ~30 ms of device time (the clock settles under
        # matrix-core load; every row below gets the same)
        "settle_ms": round(settle_ms, 2),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": "shared-QKV W8A8 projection group: x bf16 [16384,4096] quantized once to E4M3, then three "
            "E4M3 4096->4096 GEMMs with weight-scale ratios 1:0.7:0.45, bf16 outputs",
            "M": M,
            "K": K,
            "N": N,
            "projections": 3,
        },
        "pct_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "w8a16": {
            "value": round(tf16, 2),
            "unit": "TFLOP/s",
            "ms_per_step": round(ms16, 4),
            "pct_bf16_peak": round(100 * tf16 / PEAK_BF16_TFLOPS, 2),
            "settle_ms": round(settle16_ms, 2),
            "dtype": "bf16 activations x E4M3 weights (exact bf16 dequant), fp32 accumulate",
        },
        "roofline": {
            "kernel": "gemm_w8a8 (v_mfma_f32_16x16x128_f8f6f4), one grouped launch of 3 projections, "
            "each M=16384 N=4096 K=4096",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
            "avg_launch_ms": round(gemm_avg_ms, 5),
            "traffic": gemm_traffic(),
        },
    }

    if not args.no_rows:
        out["rows"] = other_rows(dev, case, x, qws, qx, ys, schedule_row=not args.no_schedule)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(out), flush=True)


def other_rows(dev, case, x, qws, qx, ys, schedule_row=True):
    rows = {}
    s_in, sw = case.input_scale, case.weight_scales
    reps = 20

    # the step as three separate GEMM calls (HIP events around each)
    evs = []
    for rep in range(reps + 5):
        fp8lin.fp8lin_quantize_static(x, s_in, out=qx)
        for i in range(3):
            e = events(2)
            e[0].record()
            fp8lin.fp8lin_gemm_w8a8(qx, qws[i], s_in, sw[i], out=ys[i])
            e[1].record()
            if rep >= 5:
                evs.append(e)
    torch.cuda.synchronize()
    t1 = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    rows["gemm_w8a8_single_launch_16384x4096x4096"] = {"ms": round(t1, 4), "tflops": round(GEMM_FLOP / t1 / 1e9, 2)}

    # grouped shared-QKV call, both modes (one quantize + one grouped GEMM launch / one grouped W8A16 launch)
    t8 = timed(lambda: fp8lin.fp8lin_qkv_shared(x, qws, sw, [s_in] * 3, fp8lin.MODE_W8A8, outs=ys, workspace=qx), reps)
    t16 = timed(lambda: fp8lin.fp8lin_qkv_shared(x, qws, sw, [s_in] * 3, fp8lin.MODE_W8A16, outs=ys), reps)
    rows["qkv_shared_w8a8"] = {"ms": round(t8, 4), "tflops": round(3 * GEMM_FLOP / t8 / 1e9, 2)}
    rows["qkv_shared_w8a16"] = {"ms": round(t16, 4), "tflops": round(3 * GEMM_FLOP / t16 / 1e9, 2)}

    # dynamic per-tensor FP8 on the same activation: amax pass + quantize with the device scale, then the
    # three projections reading that scale from device memory
    s_dev = torch.empty(1, dtype=torch.float32, device=dev)
    ws_dev = torch.empty(1, dtype=torch.int32, device=dev)
    t_qd = timed(lambda: fp8lin.fp8lin_quantize_dynamic(x, out=qx, scale=s_dev, workspace=ws_dev), reps)
    t_qs = timed(lambda: fp8lin.fp8lin_quantize_static(x, s_in, out=qx), reps)

    def step_dynamic():
        fp8lin.fp8lin_quantize_dynamic(x, out=qx, scale=s_dev, workspace=ws_dev)
        for i in range(3):
            fp8lin.fp8lin_gemm_w8a8_dev_scale(qx, qws[i], s_dev, sw[i], out=ys[i])

    t_dyn = timed(step_dynamic, reps)
    rows["dynamic_fp8_qkv_16384x4096"] = {
        "quantize_dynamic_ms": round(t_qd, 4), "quantize_static_ms": round(t_qs, 4),
        "amax_pass_gbps": round(2 * M * K / max(t_qd - t_qs, 1e-6) / 1e6, 1),
        "step_ms": round(t_dyn, 4), "step_tflops": round(3 * GEMM_FLOP / t_dyn / 1e9, 2),
    }

    # quantize at [16384, 4096]: 2 bytes in + 1 byte out per element, buffers rotated over > 512 MB
    n = M * K
    xs = rotating(lambda i: normal_bf16((M, K), 0.35, 900 + i).to(dev), 600e6, 3 * n)
    qs = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in xs]
    it = [0]

    def q_once():
        i = it[0] % len(xs)
        it[0] += 1
        fp8lin.fp8lin_quantize_static(xs[i], s_in, out=qs[i])

    tq = timed(q_once, 30)
    rows["quantize_16384x4096"] = {"ms": round(tq, 4), "gbps": round(3 * n / tq / 1e6, 1),
                                   "pct_hbm_peak": round(100 * 3 * n / tq / 1e6 / PEAK_HBM_GBPS, 2),
                                   "rotated_sets": len(xs)}
    del xs, qs

    # SwiGLU at [8192, 16384]: 4 bytes in + 1 (E4M3) or 2 (bf16) bytes out per element
    mi, inter = 8192, 16384
    n2 = mi * inter
    gs = [(normal_bf16((mi, inter), 0.45, 910 + 2 * i).to(dev), normal_bf16((mi, inter), 0.45, 911 + 2 * i).to(dev))
          for i in range(2)]
    o8 = [torch.empty((mi, inter), dtype=torch.uint8, device=dev) for _ in gs]
    o16 = torch.empty((mi, inter), dtype=torch.bfloat16, device=dev)
    it[0] = 0

    def sw8():
        i = it[0] % len(gs)
        it[0] += 1
        fp8lin.fp8lin_swiglu_2in_quant(gs[i][0], gs[i][1], 2.1 / 448, fp8lin.DT_E4M3, out=o8[i])

    def sw16():
        i = it[0] % len(gs)
        it[0] += 1
        fp8lin.fp8lin_swiglu_2in_quant(gs[i][0], gs[i][1], 1.0, fp8lin.DT_BF16, out=o16)

    ts8 = timed(sw8, 20)
    ts16 = timed(sw16, 20)
    rows["swiglu_fp8_8192x16384"] = {"ms": round(ts8, 4), "gbps": round(5 * n2 / ts8 / 1e6, 1),
                                     "pct_hbm_peak": round(100 * 5 * n2 / ts8 / 1e6 / PEAK_HBM_GBPS, 2)}
    rows["swiglu_bf16_8192x16384"] = {"ms": round(ts16, 4), "gbps": round(6 * n2 / ts16 / 1e6, 1),
                                      "pct_hbm_peak": round(100 * 6 * n2 / ts16 / 1e6 / PEAK_HBM_GBPS, 2)}

    # the same SwiGLU from binary16 gate/up (E4M3 or binary16 out)
    gh = [(g.half(), u.half()) for g, u in gs]
    o16h = torch.empty((mi, inter), dtype=torch.float16, device=dev)
    it[0] = 0

    def swh8():
        i = it[0] % len(gh)
        it[0] += 1
        fp8lin.fp8lin_swiglu_2in(gh[i][0], gh[i][1], 2.1 / 448, fp8lin.DT_E4M3, out=o8[i])

    def swh16():
        i = it[0] % len(gh)
        it[0] += 1
        fp8lin.fp8lin_swiglu_2in(gh[i][0], gh[i][1], 1.0, fp8lin.DT_F16, out=o16h)

    th8 = timed(swh8, 20)
    th16 = timed(swh16, 20)
    rows["swiglu_f16_in_8192x16384"] = {
        "fp8_out_ms": round(th8, 4), "fp8_out_gbps": round(5 * n2 / th8 / 1e6, 1),
        "f16_out_ms": round(th16, 4), "f16_out_gbps": round(6 * n2 / th16 / 1e6, 1),
    }
    del gh, o16h

    # per-head QK RMSNorm + RoPE on the group's contiguous Q and K (32 heads of 128 per token)
    hd = 128
    cq, sq = (v.to(dev) for v in rope_tables(M, hd))
    wq = norm_weight_bf16(hd, 950).to(dev)
    wk = norm_weight_bf16(hd, 951).to(dev)
    qo, ko = torch.empty_like(ys[0]), torch.empty_like(ys[1])
    t_qk = timed(lambda: fp8lin.fp8lin_qk_norm_rope(ys[0], ys[1], wq, wk, cq, sq, hd, 1e-6, q_out=qo, k_out=ko), reps)
    qk_bytes = 2 * M * N * 4 + M * hd * 4  # Q and K read and written once, plus the cos / sin tables
    rows["qk_norm_rope_16384x2x4096"] = {"ms": round(t_qk, 4), "gbps": round(qk_bytes / t_qk / 1e6, 1),
                                         "pct_hbm_peak": round(100 * qk_bytes / t_qk / 1e6 / PEAK_HBM_GBPS, 2)}

    # the same consumer fused into the grouped QKV launch's epilogue, against the two launches
    def qkv_then_norm():
        fp8lin.fp8lin_gemm_w8a8_group(qx, qws, s_in, sw, outs=ys)
        fp8lin.fp8lin_qk_norm_rope(ys[0], ys[1], wq, wk, cq, sq, hd, 1e-6, q_out=qo, k_out=ko)

    fused_outs = [qo, ko, ys[2]]
    t_sep = timed(qkv_then_norm, reps)
    t_fus = timed(lambda: fp8lin.fp8lin_qkv_w8a8_norm_rope(qx, qws, s_in, sw, wq, wk, cq, sq, 1e-6, outs=fused_outs),
                  reps)
    rows["qkv_w8a8_norm_rope_16384x4096x3x4096"] = {
        "separate_ms": round(t_sep, 4), "fused_ms": round(t_fus, 4), "speedup": round(t_sep / t_fus, 3),
        "fused_tflops": round(3 * GEMM_FLOP / t_fus / 1e9, 1),
    }
    del qo, ko, cq, sq

    # W8A16 with binary16 and float32 activations at the headline shape
    x16 = x.half()
    y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
    t_h = timed(lambda: fp8lin.fp8lin_gemm_w8a16(x16, qws[0], sw[0], out=y16), reps)
    del x16, y16
    x32 = x.float()
    y32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws32 = torch.empty(fp8lin.fp8lin_w8a16_f32_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    t_f = timed(lambda: fp8lin.fp8lin_gemm_w8a16_f32(x32, qws[0], sw[0], out=y32, workspace=ws32), reps)
    rows["w8a16_activation_dtypes_16384x4096x4096"] = {
        "f16_ms": round(t_h, 4), "f16_tflops": round(GEMM_FLOP / t_h / 1e9, 1),
        "f32_ms": round(t_f, 4), "f32_tflops": round(GEMM_FLOP / t_f / 1e9, 1),
        "f32_note": "split into three bf16 pieces (4 B in, 6 B out per value) + bf16 MFMA over 3K",
    }
    del x32, y32, ws32

    # gated-MLP GEMMs (gate/up 4096 -> 16384 on 8192 rows; down 16384 -> 4096) in both modes
    g_in = gs[0][0][:, :K].contiguous()  # any [8192, 4096] bf16 activation
    w_gu = torch.randint(0, 0x7E, (inter, K), dtype=torch.uint8, device=dev)
    w_dn = torch.randint(0, 0x7E, (K, inter), dtype=torch.uint8, device=dev)
    q_gu = fp8lin.fp8lin_quantize_static(g_in, 0.01)
    y_gu = torch.empty((mi, inter), dtype=torch.bfloat16, device=dev)
    y_dn = torch.empty((mi, K), dtype=torch.bfloat16, device=dev)
    f_gu = 2.0 * mi * inter * K
    tg8 = timed(lambda: fp8lin.fp8lin_gemm_w8a8(q_gu, w_gu, 0.01, 1e-4, out=y_gu), reps)
    tg16 = timed(lambda: fp8lin.fp8lin_gemm_w8a16(g_in, w_gu, 1e-4, out=y_gu), reps)
    td8 = timed(lambda: fp8lin.fp8lin_gemm_w8a8(o8[0], w_dn, 0.01, 1e-4, out=y_dn), reps)
    td16 = timed(lambda: fp8lin.fp8lin_gemm_w8a16(o16, w_dn, 1e-4, out=y_dn), reps)
    rows["gate_or_up_8192x16384x4096"] = {"w8a8_tflops": round(f_gu / tg8 / 1e9, 1), "w8a16_tflops": round(f_gu / tg16 / 1e9, 1)}
    rows["down_8192x4096x16384"] = {"w8a8_tflops": round(f_gu / td8 / 1e9, 1), "w8a16_tflops": round(f_gu / td16 / 1e9, 1)}
    del gs, o8, o16, y_gu, y_dn

    # gated MLP gate/up + SwiGLU at config 4 (x [8192, 4096], I = 16384): the split path (one quantize,
    # one grouped gate/up launch writing two bf16 [8192, 16384] tensors, the two-input SwiGLU reading them)
    # against the fused launch (one quantize, one GEMM whose epilogue emits the E4M3 h directly)
    c4 = config4()
    x4 = c4.x.to(dev)
    qg4 = fp8lin.fp8lin_quantize_static(c4.w_gate.to(dev), c4.s_gate)
    qu4 = fp8lin.fp8lin_quantize_static(c4.w_up.to(dev), c4.s_up)
    qx4 = torch.empty((mi, K), dtype=torch.uint8, device=dev)
    g4, u4 = (torch.empty((mi, inter), dtype=torch.bfloat16, device=dev) for _ in range(2))
    h4 = torch.empty((mi, inter), dtype=torch.uint8, device=dev)
    h4f = torch.empty_like(h4)

    def mlp_split():
        fp8lin.fp8lin_qkv_shared(x4, [qg4, qu4], [c4.s_gate, c4.s_up], [c4.input_scale] * 2, fp8lin.MODE_W8A8,
                                 outs=[g4, u4], workspace=qx4)
        fp8lin.fp8lin_swiglu_2in_quant(g4, u4, c4.s_h, fp8lin.DT_E4M3, out=h4)

    def mlp_fused():
        fp8lin.fp8lin_quantize_static(x4, c4.input_scale, out=qx4)
        fp8lin.fp8lin_gate_up_swiglu_w8a8(qx4, qg4, qu4, c4.input_scale, c4.s_gate, c4.s_up, c4.s_h, out=h4f)

    h16s = torch.empty((mi, inter), dtype=torch.bfloat16, device=dev)
    h16f = torch.empty_like(h16s)

    def mlp16_split():
        fp8lin.fp8lin_qkv_shared(x4, [qg4, qu4], [c4.s_gate, c4.s_up], [c4.input_scale] * 2, fp8lin.MODE_W8A16,
                                 outs=[g4, u4])
        fp8lin.fp8lin_swiglu_2in_quant(g4, u4, 1.0, fp8lin.DT_BF16, out=h16s)

    def mlp16_fused():
        fp8lin.fp8lin_gate_up_swiglu_w8a16(x4, qg4, qu4, c4.s_gate, c4.s_up, out=h16f)

    t_split = timed(mlp_split, reps)
    t_fused = timed(mlp_fused, reps)
    t16_split = timed(mlp16_split, reps)
    t16_fused = timed(mlp16_fused, reps)
    torch.cuda.synchronize()
    f_mlp = 2 * f_gu
    rows["gated_mlp_gate_up_swiglu_8192x4096x16384"] = {
        "split_ms": round(t_split, 4), "fused_ms": round(t_fused, 4), "speedup": round(t_split / t_fused, 3),
        "fused_tflops": round(f_mlp / t_fused / 1e9, 1), "split_tflops": round(f_mlp / t_split / 1e9, 1),
        "fused_equals_split": bool(torch.equal(h4, h4f)),
        "w8a16_split_ms": round(t16_split, 4), "w8a16_fused_ms": round(t16_fused, 4),
        "w8a16_speedup": round(t16_split / t16_fused, 3),
        "w8a16_fused_equals_split": bool(torch.equal(h16s.view(torch.int16), h16f.view(torch.int16))),
    }
    del x4, qg4, qu4, qx4, g4, u4, h4, h4f, h16s, h16f, c4

    # 4096 -> 4096 projection at 1024, 2048 and 8192 rows. Where 256 x 256 tiles would keep at most 60% of
    # the CUs busy the library runs 128 x 128 tiles; at 1024 rows the split-K calls on 256 x 256 tiles are
    # timed beside them for comparison.
    c2 = config2()
    x2 = c2.x.to(dev)
    qw2 = fp8lin.fp8lin_quantize_static(c2.w.to(dev), c2.weight_scale)
    q2 = fp8lin.fp8lin_quantize_static(x2, c2.input_scale)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    for m in (1024, 2048, 8192):
        y2 = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
        f = 2.0 * m * N * K
        a = timed(lambda: fp8lin.fp8lin_gemm_w8a8(q2[:m], qw2, c2.input_scale, c2.weight_scale, out=y2), reps)
        b = timed(lambda: fp8lin.fp8lin_gemm_w8a16(x2[:m], qw2, c2.weight_scale, out=y2), reps)
        big_tiles = ((m + 255) // 256) * (N // 256)
        row = {"tiles": "128x128" if 5 * big_tiles <= 3 * cus else "256x256",
               "w8a8_tflops": round(f / a / 1e9, 1), "w8a8_pct_fp8_peak": round(100 * f / a / 1e9 / PEAK_FP8_TFLOPS, 2),
               "w8a16_tflops": round(f / b / 1e9, 1),
               "w8a16_pct_bf16_peak": round(100 * f / b / 1e9 / PEAK_BF16_TFLOPS, 2)}
        if m < 8192:
            # the same calls replayed from a captured graph: at 17-60 us per kernel the host's launch time
            # between eager calls shows in the rows above
            q2m, x2m = q2[:m], x2[:m]
            ag = timed_graph(lambda: fp8lin.fp8lin_gemm_w8a8(q2m, qw2, c2.input_scale, c2.weight_scale, out=y2),
                             reps)
            bg = timed_graph(lambda: fp8lin.fp8lin_gemm_w8a16(x2m, qw2, c2.weight_scale, out=y2), reps)
            row["graph_replay"] = {
                "calls_per_graph": 20,
                "w8a8_tflops": round(f / ag / 1e9, 1),
                "w8a8_pct_fp8_peak": round(100 * f / ag / 1e9 / PEAK_FP8_TFLOPS, 2),
                "w8a16_tflops": round(f / bg / 1e9, 1),
                "w8a16_pct_bf16_peak": round(100 * f / bg / 1e9 / PEAK_BF16_TFLOPS, 2)}
        if m == 1024:
            ws_sk = torch.empty(4 * m * K * 4, dtype=torch.uint8, device=dev)
            c = timed(lambda: fp8lin.fp8lin_gemm_w8a8_splitk(q2[:m], qw2, c2.input_scale, c2.weight_scale,
                                                             splits=2, out=y2, workspace=ws_sk), reps)
            d = timed(lambda: fp8lin.fp8lin_gemm_w8a16_splitk(x2[:m], qw2, c2.weight_scale, splits=4, out=y2,
                                                              workspace=ws_sk), reps)
            row["splitk_256x256"] = {"w8a8_2_splits_tflops": round(f / c / 1e9, 1),
                                     "w8a16_4_splits_tflops": round(f / d / 1e9, 1)}
        rows["proj_%dx4096x4096" % m] = row

    # step policy: host call per transformer forward
    pol = step_policy_of_workload()
    trace = [fp8lin.fp8lin_step_policy(pol, 0, i, 8) for i in range(8)]
    t0 = time.perf_counter()
    for i in range(10000):
        fp8lin.fp8lin_step_policy(pol, 0, i % 8, 8)
    rows["step_policy"] = {"us_per_call_incl_python": round((time.perf_counter() - t0) * 100, 3),
                           "trace_8": "".join("8" if t == fp8lin.MODE_W8A8 else "6" for t in trace)}
    if schedule_row:
        rows["schedule_cfg5"] = schedule_cfg5(dev, pol)
    return rows


def step_policy_of_workload():
    """The denoising policy of the schedule workload: first 3 and last 3 steps W8A16, the rest W8A8."""
    return fp8lin.policy_from_json({"schema_version": 1, "type": "first_last_steps", "index_space": "scheduler_step",
                                    "default_mode": "w8a8", "overlap": "a16", "first_steps": 3, "last_steps": 3,
                                    "reasoner": "a16"})


def schedule_cfg5(dev, pol):
    """The 8-step denoising schedule: 4 blocks x 2 CFG passes x 8 steps at 16384 rows, policy first 3 / last 3."""
    from w8a16_linear_layers_amd import schedule
    from workloads import config5, config5_step_input

    m, hidden, inter, nblocks, steps = 16384, 4096, 16384, 4, 8
    log("schedule row: building 4 synthetic blocks (calibration forward on the GPU)")
    cases = config5(num_blocks=nblocks, hidden=hidden, inter=inter, cal_rows=256, device=dev)
    q = lambda w, s: fp8lin.fp8lin_quantize_static(w.to(dev), s)  # noqa: E731
    blocks = [
        schedule.BlockWeights(
            [q(w, s) for w, s in zip(c.w_qkv, c.s_qkv)], c.s_qkv, c.s_in_qkv,
            q(c.w_out, c.s_out), c.s_out, c.s_in_out,
            q(c.w_gate, c.s_gate), q(c.w_up, c.s_up), c.s_gate, c.s_up, c.s_in_mlp,
            q(c.w_down, c.s_down), c.s_down, c.s_h,
        )
        for c in cases
    ]
    del cases
    buf = schedule.Buffers(m, hidden, inter, dev)
    log("schedule row: generating the 16 per-pass inputs")
    inputs = {(st, b): config5_step_input(st, b, m, hidden).to(dev) for st in range(steps) for b in range(2)}
    step_ev = {st: events(2) for st in range(steps)}

    def hook(st, mode, done):
        step_ev[st][1 if done else 0].record()

    def run(fused):
        return schedule.run_schedule(blocks, pol, steps, lambda st, b: inputs[(st, b)], buf, fused_mlp=fused,
                                     step_hook=hook)

    run(True)  # warm-up pass
    torch.cuda.synchronize()
    # the schedule as it runs by default: gate/up + SwiGLU in one fused launch on every step
    trace = run(True)
    torch.cuda.synchronize()
    step_ms = [step_ev[st][0].elapsed_time(step_ev[st][1]) for st in range(steps)]
    ms = step_ev[0][0].elapsed_time(step_ev[steps - 1][1])
    # the same schedule with the split gate/up launch and a separate SwiGLU kernel
    run(False)
    torch.cuda.synchronize()
    ms_split = step_ev[0][0].elapsed_time(step_ev[steps - 1][1])
    flop_pass = 2.0 * m * hidden * (4 * hidden + 3 * inter)  # QKV + out + gate/up + down of one block
    flop_step = flop_pass * nblocks * 2
    flop = flop_step * steps
    w8 = [t for st, t in enumerate(step_ms) if trace[st] == fp8lin.MODE_W8A8]
    w16 = [t for st, t in enumerate(step_ms) if trace[st] != fp8lin.MODE_W8A8]
    kind = lambda ts: {"steps": len(ts), "ms_per_step": round(float(np.mean(ts)), 3),  # noqa: E731
                       "tflops": round(flop_step / float(np.mean(ts)) / 1e9, 1)} if ts else None
    return {
        "ms": round(ms, 2),
        "tflops": round(flop / ms / 1e9, 1),
        "mlp": "fused gate/up + SwiGLU",
        "ms_split_mlp": round(ms_split, 2),
        "tflop": round(flop / 1e12, 1),
        "trace": "".join("8" if t == fp8lin.MODE_W8A8 else "6" for t in trace),
        "w8a8_steps": kind(w8),
        "w8a16_steps": kind(w16),
        "step_ms": [round(t, 3) for t in step_ms],
    }


if __name__ == "__main__":
    main()
