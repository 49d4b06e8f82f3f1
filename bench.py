#!/usr/bin/env python3
"""Fused MoE layer benchmark on one MI355X.

A step is one moe_fused_forward call (routing -> GEMM-1 + SwiGLU -> GEMM-2 +
routing weight -> combine) over the synthetic workload, inputs resident in
HBM.  The default workload is the largest single-GPU one: 8192 tokens of the
DeepSeek-shaped FP8 layer (7168/2048, 32 experts, top-2, two experts with 30%
of the assignments each, 16 empty).  W untimed warmup steps, then K timed
steps, each bracketed by HIP events on the stream the library launches on,
with the L2s and the 256 MB Infinity Cache flushed before each step outside
its events (cold); the same steps without the flush give the warm figures.
The line reports the cold p50 step time (ms_per_step), TFLOP/s at that p50
(algorithmic FLOPs = 6*d_h*d_e per valid assignment), the dominant kernel's
roofline fraction from its mean dispatch duration, and the CPU oracle timed on
a bounded sample.

The weights are rewritten once, before any timing, into the packed tile order
(moe_pack_weights), as a deployment does when it loads them; ``--weights
row-major`` times the layer on the weights as given instead.

``--launch single`` times the single-launch form (the whole layer in one
persistent kernel, moe_dims.launch = MOE_LAUNCH_SINGLE); the roofline is then
the whole layer's, that kernel being the only one.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--weights packed|row-major] [--no-cpu]
                    [--launch multi|single]
    python bench.py --pass backward --config qwen_bf16   (the backward with recompute)
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused MoE layer p50 µs + TFLOP/s (% MFMA/HBM roofline), 1 MI355X"
PEAK_HBM_GBS = 8000.0
# dense MFMA: bf16 (F32ACT and INT8 tokens run bf16 MFMA), fp8
PEAK_TFLOPS = {0: 2500.0, 1: 2500.0, 2: 5000.0, 3: 5000.0, 4: 2500.0}
DTYPE = {0: "bf16", 1: "bf16", 2: "fp8_e4m3", 3: "mxfp8_e4m3", 4: "bf16 (int8 tokens)"}
DEFAULT_CONFIG = "ds_fp8_8192"


def gemm1_alg_bytes(w):
    """Bytes GEMM-1 must move once: active experts' W1 (+ scales), x (+ scales), h (+ scales)."""
    from skew_aware_grouped_amd import workloads as W
    a = w.active_experts()
    fp8 = w.mode in (W.MODE_FP8, W.MODE_MXFP8)
    wb = 1 if fp8 else 2
    xb = 1 if fp8 else {W.MODE_F32ACT: 4, W.MODE_BF16: 2, W.MODE_INT8: 1}[w.mode]
    nv = w.valid_assignments()
    b = a * 2 * w.d_e * w.d_h * wb + w.T * w.d_h * xb + nv * w.d_e * wb
    if w.mode == W.MODE_FP8:  # fp32 scales per 128x128 block (W1), per row per 128 (x, h)
        b += a * (2 * w.d_e // 128) * (w.d_h // 128) * 4 + w.T * (w.d_h // 128) * 4 + nv * (w.d_e // 128) * 4
    if w.mode == W.MODE_MXFP8:  # one E8M0 byte per row per 32 values
        b += a * 2 * w.d_e * (w.d_h // 32) + w.T * (w.d_h // 32) + nv * (w.d_e // 32)
    if w.mode == W.MODE_INT8:  # one fp32 scale per token
        b += w.T * 4
    return float(b)


# The sources each timed kernel is compiled from: a traffic record stays valid
# while these are unchanged.
KERNEL_SOURCES = {
    "layer_kernel": ["moe_layer.hip", "moe_gemm_task.h", "moe_wave.h", "moe_internal.h"],
    "route_kernel": ["moe_route.hip", "moe_wave.h", "moe_internal.h"],
}
GEMM_SOURCES = ["moe_gemm.hip", "moe_gemm_task.h", "moe_internal.h"]


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(kernel, GEMM_SOURCES):
        with open(os.path.join(ROOT, "skew_aware_grouped_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, weights):
    """HBM-side bytes per launch from the committed counter summary
    (profiles/, FETCH_SIZE + WRITE_SIZE scaled by a copy of known size), or
    None when no record exists or the kernel sources changed since it was taken."""
    import glob
    src = kernel_source_hash(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                line = line.strip()
                if not line.startswith("traffic_record:"):
                    continue
                rec = json.loads(line[len("traffic_record:"):])
                if rec.get("kernel") == kernel and rec.get("workload") == workload and \
                        rec.get("weights", "row-major") == weights and rec.get("source_sha256_16") == src:
                    return float(rec["traffic_bytes"])
    return None


def cpu_model():
    """The host CPU's model name, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, target_s=12.0):
    """The oracle as it stands, on a bounded sample of the workload: a token
    subset when the whole batch would take longer than ~target_s, otherwise the
    whole batch repeated until ~target_s of CPU work has run."""
    from oracle import moe_oracle
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    rng = np.random.default_rng(0)
    # calibrate on a few tokens, then size the sample to ~target_s
    probe = rng.choice(w.T, size=min(16, w.T), replace=False)
    t0 = time.perf_counter()
    moe_oracle.forward(w, rows=probe)
    dt = max(time.perf_counter() - t0, 1e-6)
    n = int(min(w.T, max(len(probe), len(probe) * target_s / dt)))
    rows = np.sort(rng.choice(w.T, size=n, replace=False))
    reps = 1 if n < w.T else max(1, int(round(target_s / (dt * w.T / len(probe)))))
    t0 = time.perf_counter()
    for _ in range(reps):
        moe_oracle.forward(w, rows=rows)
    dt = time.perf_counter() - t0
    sub_ids = w.topk_ids[rows]
    nv = int(((sub_ids >= 0) & (sub_ids < w.E)).sum())
    flops = 6.0 * w.d_h * w.d_e * nv * reps
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n} of {w.T} tokens ({nv} assignments) of {w.name}, {reps} pass(es), {dt:.2f} s, "
                      f"fp32 C oracle with OpenMP over tokens",
            "seconds": round(dt, 3)}


def copy_calibration(mb):
    """A plain device-to-device copy of a known size, for scaling the HBM byte
    counters of a profiler run (FETCH_SIZE / WRITE_SIZE read for this copy
    against the bytes it must move)."""
    import torch
    n = mb * (1 << 20)
    a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def backward_alg(w):
    """FLOPs and bytes the backward with recompute must do: per valid assignment
    16*d_h*d_e FLOPs (recomputed gate/up 4, q 2, dX 4, dW1 4, dW2 2); bytes: the
    active experts' W1 and W2 read once (bf16), dW1 and dW2 of every expert
    written (fp32), x and dout read, dx written (fp32), ids, weights and their
    gradient."""
    nv = w.valid_assignments()
    flops = 16.0 * w.d_h * w.d_e * nv
    wb = 3 * w.d_h * w.d_e
    byts = w.active_experts() * wb * 2 + w.E * wb * 4 + w.T * w.d_h * (2 + 2 + 4) + w.T * w.k * 12
    return flops, float(byts)


def bench_backward(args):
    """The backward pass with recompute (moe_fused_backward, BF16) on one
    workload: cold and warm p50 of K calls between events on the library's
    stream, TFLOP/s, and the whole pass against the HBM roofline (its bytes are
    dominated by writing fp32 weight gradients).  A correctness gate against
    the backward oracle runs first."""
    import torch
    from oracle import moe_oracle
    from skew_aware_grouped_amd import device, moe, workloads as W
    torch.cuda.set_device(0)
    w = W.config(args.config)
    if w.mode != W.MODE_BF16:
        print("bench.py: the backward runs BF16 workloads (e.g. --config qwen_bf16)", file=sys.stderr)
        sys.exit(2)
    d = device.upload(w)
    rng = np.random.default_rng(7)
    dout_bits = W.to_bf16_bits(rng.standard_normal((w.T, w.d_h), dtype=np.float32))
    dout = torch.from_numpy(dout_bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    dims = moe.make_dims(d["x"], d["topk_ids"], d["w1"])
    ws = torch.empty(moe.moe_backward_workspace_bytes(dims), dtype=torch.uint8, device="cuda:0")
    args_b = (d["x"], d["topk_ids"], d["topk_w"], d["w1"], d["w2"], dout)
    got = moe.fused_backward(*args_b, workspace=ws)
    torch.cuda.synchronize()
    ref = moe_oracle.backward(w, dout_bits)
    errs = {n: float(np.abs(g.cpu().numpy() - r).max() / max(np.abs(r).max(), 1e-30))
            for n, g, r in zip(("dx", "dw1", "dw2", "dtopk_w"), got, ref)}
    if not all(v <= 1e-2 for v in errs.values()):
        print(f"bench.py: backward correctness gate failed {errs}", file=sys.stderr)
        sys.exit(1)
    for _ in range(args.warmup):
        moe.fused_backward(*args_b, workspace=ws)
    stream = torch.cuda.current_stream()
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")

    def timed(n, cold):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in evs:
            if cold:
                flush.sum()
            a.record(stream)
            moe.fused_backward(*args_b, workspace=ws, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    cold_ms = timed(args.steps, True)
    warm_ms = timed(args.steps, False)
    p50 = float(np.median(cold_ms))
    flops, byts = backward_alg(w)
    gbs = byts / (p50 * 1e-3) / 1e9
    res = {
        "metric": "fused MoE layer backward with recompute p50 µs + TFLOP/s (% HBM roofline), 1 MI355X",
        "value": round(flops / (p50 * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(p50, 5), "ms_per_step_is": "cold p50 (caches flushed before each step)",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "tokens": w.T, "experts": w.E, "top_k": w.k,
                   "d_hidden": w.d_h, "d_expert": w.d_e, "active_experts": w.active_experts()},
        "p50_us": round(p50 * 1e3, 2), "warm_p50_us": round(float(np.median(warm_ms)) * 1e3, 2),
        "gflop": round(flops / 1e9, 4), "alg_mb": round(byts / 1e6, 3),
        "roofline": {"kernel": "whole backward pass", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
        "gate_normwise_err": {k: round(v, 6) for k, v in errs.items()},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--weights", choices=["packed", "row-major"], default="packed",
                    help="weight layout the layer reads (packing happens once, outside the timed region)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline leg")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward"], default="forward",
                    help="backward: time moe_fused_backward (BF16 workloads, e.g. --config qwen_bf16)")
    ap.add_argument("--launch", choices=["multi", "single"], default="multi",
                    help="single: the whole layer as one persistent kernel (BF16/FP8/MXFP8, <= 2048 assignments)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain copy of this many MiB (for scaling profiler byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this layer runs on one GPU; --gpus above 1 is not supported (the multi-GPU expert-"
              "parallel path is a design, not a build).", file=sys.stderr)
        sys.exit(2)

    if args.which == "backward":
        bench_backward(args)
        return
    import torch
    from skew_aware_grouped_amd import device, moe, workloads as W

    torch.cuda.set_device(0)
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb)
        return
    w = W.config(args.config)
    single = args.launch == "single"
    launch = moe.MOE_LAUNCH_SINGLE if single else moe.MOE_LAUNCH_MULTI
    d = device.upload(w, packed=args.weights == "packed")
    dims = moe.make_dims(d["x"], d["topk_ids"], d["w1"], weight_layout=d["weight_layout"], x_scale=d["x_scale"],
                         launch=launch)
    ws = moe.workspace_for(dims, "cuda:0")

    def run(**kw):
        return device.run(d, out=out, workspace=ws, launch=launch, **kw)
    odt = torch.float32 if w.mode == W.MODE_F32ACT else torch.bfloat16
    out = torch.empty(w.T, w.d_h, dtype=odt, device="cuda:0")

    # correctness gate before timing: a few sampled rows against the oracle
    from oracle import moe_oracle
    run()
    torch.cuda.synchronize()
    rows = sorted(set(np.random.default_rng(1).choice(w.T, size=min(8, w.T), replace=False).tolist()))
    acc, _ = moe_oracle.forward(w, rows=rows)
    got = device.out_to_f64(out)[rows]
    gate_err = float(np.abs(got - acc).max() / np.abs(acc).max())
    tol = 3e-2 if w.mode in (W.MODE_FP8, W.MODE_MXFP8) else 1e-2
    if not gate_err <= tol:
        print(f"bench.py: correctness gate failed (normwise err {gate_err:.3e} > {tol})", file=sys.stderr)
        sys.exit(1)

    for _ in range(args.warmup):
        run()
    stream = torch.cuda.current_stream()
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")

    def timed_steps(n, cold):
        """n layer calls, each between two events on the library's stream (no
        event between its kernels); cold: a read of a 1 GiB buffer before each
        call, outside its events, leaves the L2s and the 256 MB Infinity Cache
        holding other (clean) lines."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in evs:
            if cold:
                flush.sum()
            a.record(stream)
            run(stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs]), time.perf_counter() - t0

    def dispatch_steps(n, cold):
        """n calls of the kernel-timing variant: each of the four dispatches
        records its own start and end (the durations a kernel trace reports)."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(n)]
        for i in range(n):
            if cold:
                flush.sum()
            run(stream=stream, events=ev[i])
        torch.cuda.synchronize()
        return np.array([[e[2 * j].elapsed_time(e[2 * j + 1]) for j in range(4)] for e in ev])

    cold_ms, wall = timed_steps(args.steps, cold=True)
    warm_ms, _ = timed_steps(args.steps, cold=False)
    # per-kernel durations over as many cold as warm dispatches: every launch
    # of the run is one or the other, so the mean is the one a kernel trace of
    # the whole command averages to
    stage_ms = np.concatenate([dispatch_steps(args.steps, cold=True), dispatch_steps(args.steps, cold=False)])
    del flush
    p50 = float(np.median(cold_ms))
    warm_p50 = float(np.median(warm_ms))
    flops = W.flops(w)
    alg_bytes = W.algorithmic_bytes(w)
    tflops = flops / (p50 * 1e-3) / 1e12
    names = ["layer_kernel"] if single else ["route", "gemm1_swiglu", "gemm2_weight", "combine"]
    stages = {n: round(float(np.mean(stage_ms[:, j])) * 1e3, 2) for j, n in enumerate(names)}
    layer_gbs = alg_bytes / (p50 * 1e-3) / 1e9
    # dominant kernel: GEMM-1 (gate|up + SwiGLU), two thirds of the weights and
    # FLOPs; in the single launch, the one kernel and the whole layer's work
    kj = 0 if single else 1
    # the FP8 (MXFP8) GEMM-1 of batches from 2048 (4096) assignments is an
    # 8-wave kernel of its own (the library's fp8_wide rule)
    min_n = 4096 if w.mode == W.MODE_MXFP8 else 2048
    wide = (w.mode in (W.MODE_FP8, W.MODE_MXFP8) and w.T * w.k >= min_n and w.T * w.d_h < 2 ** 31
            and 2 * w.d_e * w.d_h < 2 ** 31)
    wide_name = "gemm1_fp8_kernel" if w.mode == W.MODE_FP8 else "gemm1_mxfp8_kernel"
    kname = "layer_kernel" if single else (wide_name if wide else "gemm1_kernel")
    k_us = float(np.mean(stage_ms[:, kj])) * 1e3
    g1_bytes = alg_bytes if single else gemm1_alg_bytes(w)
    g1_flops = flops if single else 4.0 * w.d_h * w.d_e * w.valid_assignments()
    k_gbs = g1_bytes / (k_us * 1e-6) / 1e9
    k_tflops = g1_flops / (k_us * 1e-6) / 1e12
    peak_f = PEAK_TFLOPS[w.mode]
    if g1_flops / (peak_f * 1e12) > g1_bytes / (PEAK_HBM_GBS * 1e9):
        roof = {"kernel": kname, "bound": "mfma", "achieved": round(k_tflops, 2), "peak": peak_f,
                "unit": "TFLOP/s", "frac": round(k_tflops / peak_f, 4)}
    else:
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(k_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(k_gbs / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": measured_traffic(kname, w.name, args.weights), "alg_bytes_per_launch": g1_bytes,
                 "alg_flops_per_launch": g1_flops, "avg_launch_us": round(k_us, 2),
                 "avg_launch_source": f"mean of {len(stage_ms)} dispatch-event durations on the library's "
                                      f"stream ({args.steps} after a cache flush, {args.steps} warm)",
                 "avg_launch_us_cold": round(float(np.mean(stage_ms[:args.steps, kj])) * 1e3, 2),
                 "avg_launch_us_warm": round(float(np.mean(stage_ms[args.steps:, kj])) * 1e3, 2)})
    res = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(p50, 5),
        "ms_per_step_is": "cold p50 (caches flushed before each step)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE[w.mode],
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "experts": w.E, "top_k": w.k, "d_hidden": w.d_h,
                   "d_expert": w.d_e, "active_experts": w.active_experts(),
                   "valid_assignments": w.valid_assignments(), "routing": str(w.meta.get("routing")),
                   "weight_layout": args.weights, "launch": args.launch},
        "p50_us": round(p50 * 1e3, 2),
        "p10_us": round(float(np.percentile(cold_ms, 10)) * 1e3, 2),
        "p90_us": round(float(np.percentile(cold_ms, 90)) * 1e3, 2),
        "warm_p50_us": round(warm_p50 * 1e3, 2),
        "warm_p10_us": round(float(np.percentile(warm_ms, 10)) * 1e3, 2),
        "warm_p90_us": round(float(np.percentile(warm_ms, 90)) * 1e3, 2),
        "warm_tflops": round(flops / (warm_p50 * 1e-3) / 1e12, 3),
        "wall_us_per_step_cold_incl_flush": round(wall / args.steps * 1e6, 2),
        "gflop": round(flops / 1e9, 4),
        "alg_mb": round(alg_bytes / 1e6, 3),
        "layer_gbs": round(layer_gbs, 1),
        "layer_roofline_frac": round(max(layer_gbs / PEAK_HBM_GBS, tflops / PEAK_TFLOPS[w.mode]), 4),
        "stage_us": stages,
        "gate_normwise_err": round(gate_err, 6),
        "roofline": roof,
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
