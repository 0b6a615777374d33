#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 linear layer on one MI355X.

One step is one full layer call (svdq_linear_w4a4: the fused activation
kernel, then the W4xA4 GEMM with its low-rank / bias epilogue) on one batch
of seeded synthetic activations, inputs resident in HBM.  The timed steps
replay a HIP graph of the same library calls (no host launch gaps); the
eager per-call loop is timed too and reported beside it.  Workload: the
FLUX-scale projection M 4096 x K 3072 -> N 12288, rank 32, INT4 groups of 64,
bf16 activations and output.  Weights are quantized once, offline, by the
library's own svdq_quantize_weights.

Prints one JSON line: TOPS = 2 M N K / (time per step), the roofline of the
dominant kernel (the GEMM) measured with HIP events on the launch stream, and
the CPU oracle's throughput on a bounded sample of the same workload.  The
same line carries, under "other_paths", the NVFP4 precision at the MLP
up-projection shape and the AWQ W4A16 layer at M = 1, 16, 4608.

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-other-paths]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_FP8_TOPS = 5000.0          # MI355X dense FP8 / INT8 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0        # dense fp16 / bf16 MFMA
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP4_TFLOPS = 10100.0       # dense fp4 / fp6 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--nbuf", type=int, default=4, help="distinct X / Y buffers rotated")
    ap.add_argument("--no-other-paths", action="store_true",
                    help="skip the NVFP4 and AWQ W4A16 measurements")
    ap.add_argument("--other-steps", type=int, default=50)
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first run a plain device copy of this many MiB three times "
                         "(a known-size kernel to calibrate rocprofv3 byte counters)")
    return ap.parse_args()


def gemm_source_sha():
    h = hashlib.sha256()
    for f in ("gemm_int4.hip", "internal.h"):
        with open(os.path.join(ROOT, "w4a4_quantized_diffusion_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(launch_units):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "gemm_int4_flagship_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_sha") != gemm_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(M, K, N, R, seconds):
    """The oracle forward (INT4 quantization of the activations, exact group
    products, fp64 scaled accumulation, bf16 low-rank branch) on a bounded
    sample of rows of the same workload, timed on the host cores."""
    import numpy as np
    from oracle import svdq as O
    from oracle import formats as F
    from w4a4_quantized_diffusion_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    r = synth.random_int4_layer(N, K, R, seed=0)
    lay = dict(q=O.unpack_int4(r["wcodes"]), sW=r["sW"], smooth=r["smooth"],
               lora_down=F.bf16_to_f32(r["lora_down_bits"]).astype(np.float64),
               lora_up=F.bf16_to_f32(r["lora_up_bits"]).astype(np.float64))
    x = synth.layer(M, K, 16, 0, seed=0)["x"]
    rows = 8
    t = 0.0
    while True:                      # grow the sample until it is ~1/8 of the budget
        t0 = time.perf_counter()
        O.linear_w4a4(x[:rows], lay)
        t = time.perf_counter() - t0
        if t > seconds / 8 or rows >= M:
            break
        rows = min(M, rows * 2)
    rows = min(M, max(rows, int(rows * (seconds / max(t, 1e-9)))))
    t0 = time.perf_counter()
    O.linear_w4a4(x[:rows], lay)
    t = time.perf_counter() - t0
    tops = 2.0 * rows * N * K / t / 1e12
    return {"value": tops, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {M} rows of the same layer (full K={K}, N={N}, rank {R}), "
                      f"{t:.1f} s, numpy/BLAS on the host"}


def time_calls(fn, steps, warmup=3):
    """Per-call durations (seconds) of fn(i), HIP events on the current
    stream around each call."""
    import numpy as np
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs]) * 1e-3


def time_loop(fn, steps, warmup=3):
    """Average duration (seconds) of fn(i) issued back to back, HIP events
    on the current stream around the whole loop.  For kernels of a few
    microseconds an event pair around each call adds its own overhead; the
    loop average is the rate at which the stream runs them."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / steps


def other_paths(steps):
    """The NVFP4 precision at the MLP up-projection shape (M 4608, K 3072 ->
    N 12288, rank 32), the INT4 MLP down-projection with the GELU fused in
    (M 4608, K 12288 -> N 3072) and the AWQ W4A16 layer (K 3072 -> N 12288) at M = 1,
    16 and 4608: seeded synthetic tensors, weights quantized by the library
    (the down-projection's INT4 layer drawn directly), per-kernel HIP-event
    times.  Weight-streaming cases rotate enough weight copies (> 512 MB)
    that the 256 MB last-level cache cannot hold them."""
    import numpy as np
    import torch
    from w4a4_quantized_diffusion_amd import svdq, synth, layout
    dev = torch.device("cuda:0")
    res = {}

    # NVFP4, MLP up-projection
    M, K, N, R = 4608, 3072, 12288, 32
    s = synth.layer(M, K, N, R, seed=0, workload="mlp_fp4")
    x = torch.from_numpy(s["x"]).to(dev).to(torch.bfloat16)
    bias = torch.from_numpy(s["b"]).to(dev).to(torch.bfloat16)
    amax = svdq.svdq_act_absmax(x)
    lay = svdq.svdq_quantize_weights(torch.from_numpy(s["w"]).to(dev), amax, R, "nvfp4")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(svdq.svdq_workspace_bytes(M, K, R, "nvfp4"), dtype=torch.uint8, device=dev)
    codes, scales, lr = svdq.workspace_views(ws, M, K, R, "nvfp4")
    # back-to-back loops after a warm-up loop of the same length (the clock
    # ramps up under load); per-call HIP-event brackets beside them
    lin = lambda i: svdq.svdq_linear_w4a4(x, lay, bias, workspace=ws, Y=y)
    act = lambda i: svdq.svdq_act_quantize(x, lay, codes, scales, lr)
    gem = lambda i: svdq.svdq_gemm_w4a4(codes, scales, lr, lay, bias, Y=y)
    t_lin_loop = time_loop(lin, steps, warmup=steps)
    t_act_loop = time_loop(act, steps, warmup=steps)
    t_gem_loop = time_loop(gem, steps, warmup=steps)
    t_act = time_calls(act, steps)
    t_gem = time_calls(gem, steps)
    ops = 2.0 * M * N * K
    act_bytes = M * K * 2 + M * K // 2 + M * K // 16 + M * R * 2 + K * 4 + R * K * 2
    res["nvfp4_mlp_up"] = {
        "workload": "NVFP4 (E2M1 b16, E4M3 block scales), rank 32, M 4608 x K 3072 -> N 12288",
        "linear_us": round(t_lin_loop * 1e6, 2),
        "TOPS": round(ops / t_lin_loop / 1e12, 1),
        "timing": "back-to-back loop averages",
        "gemm_nvfp4": {"avg_us": round(t_gem_loop * 1e6, 2),
                       "per_call_bracket_us": round(float(t_gem.mean()) * 1e6, 2),
                       "TFLOP/s": round(ops / t_gem_loop / 1e12, 1), "bound": "mfma (f16)",
                       "frac_f16_peak": round(ops / t_gem_loop / 1e12 / PEAK_F16_TFLOPS, 4),
                       "frac_fp4_peak": round(ops / t_gem_loop / 1e12 / PEAK_FP4_TFLOPS, 4)},
        "act_quant_nvfp4": {"avg_us": round(t_act_loop * 1e6, 2),
                            "per_call_bracket_us": round(float(t_act.mean()) * 1e6, 2),
                            "timing": "back-to-back loop average",
                            "algorithmic_bytes": act_bytes,
                            "GB/s": round(act_bytes / t_act_loop / 1e9, 1),
                            "frac_hbm": round(act_bytes / t_act_loop / 1e9 / PEAK_HBM_GBS, 4)},
    }
    del x, lay, y, ws, codes, scales, lr
    torch.cuda.empty_cache()

    # INT4 MLP down-projection with the GELU fused into the activation pass
    M, K, N, R = 4608, 12288, 3072, 32
    mw = synth.WORKLOADS["mlp"]
    x = torch.from_numpy(synth.activations(M, K, 0, mw, 0)).to(dev).to(torch.bfloat16)
    r = synth.random_int4_layer(N, K, R, 0, "mlp")
    lay = dict(rank=R, prec=svdq.INT4, N=N, K=K, smooth=torch.from_numpy(r["smooth"]).to(dev),
               lora_down=torch.from_numpy(r["lora_down_bits"].view("int16")).to(dev),
               lora_up=torch.from_numpy(r["lora_up_bits"].view("int16")).to(dev),
               wcodes=torch.from_numpy(layout.int4_to_device(r["wcodes"])).to(dev),
               wscales=torch.from_numpy(np.ascontiguousarray(r["sW"].T)).to(dev),
               w_tensor_scale=torch.ones(1, device=dev), x_tensor_scale=torch.ones(1, device=dev))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(svdq.svdq_workspace_bytes(M, K, R), dtype=torch.uint8, device=dev)
    codes, scales, lr = svdq.workspace_views(ws, M, K, R)
    t_lin_g = time_loop(lambda i: svdq.svdq_linear_w4a4_gelu(x, lay, workspace=ws, Y=y), steps,
                        warmup=steps)
    t_lin_p = time_loop(lambda i: svdq.svdq_linear_w4a4(x, lay, workspace=ws, Y=y), steps,
                        warmup=steps)
    t_act_g = time_loop(lambda i: svdq.svdq_act_quantize_gelu(x, lay, codes, scales, lr), steps,
                        warmup=steps)
    t_act_p = time_loop(lambda i: svdq.svdq_act_quantize(x, lay, codes, scales, lr), steps,
                        warmup=steps)
    ops = 2.0 * M * N * K
    act_bytes = M * K * 2 + M * K // 2 + M * (K // 64) * 4 + M * R * 2 + K * 4 + R * K * 2
    res["int4_mlp_down_gelu"] = {
        "workload": "INT4 g64, rank 32, GELU fused into the activation pass, "
                    "M 4608 x K 12288 -> N 3072",
        "timing": "back-to-back loop averages",
        "linear_us": round(t_lin_g * 1e6, 2),
        "TOPS": round(ops / t_lin_g / 1e12, 1),
        "linear_without_gelu_us": round(t_lin_p * 1e6, 2),
        "act_quant_gelu_us": round(t_act_g * 1e6, 2),
        "act_quant_us": round(t_act_p * 1e6, 2),
        "act_quant_gelu_frac_hbm": round(act_bytes / t_act_g / 1e9 / PEAK_HBM_GBS, 4),
        "unfused_gelu_pass_bytes": 2 * M * K * 2,
    }
    # the same layer with a rank-16 LoRA adapter folded into its 16-bit branch
    RL = 16
    a, b = synth.lora_adapter(N, K, RL, 0)
    at = torch.from_numpy(a).to(dev).to(torch.bfloat16)
    bt = torch.from_numpy(b).to(dev).to(torch.bfloat16)
    lay_l = svdq.svdq_fold_lora(lay, at, bt, 1.0)
    ws_l = torch.empty(svdq.svdq_workspace_bytes(M, K, lay_l["rank"]), dtype=torch.uint8,
                       device=dev)
    t_fold = time_loop(lambda i: svdq.svdq_fold_lora(lay, at, bt, 1.0), 20, warmup=5)
    t_lin_l = time_loop(lambda i: svdq.svdq_linear_w4a4(x, lay_l, workspace=ws_l, Y=y), steps,
                        warmup=steps)
    fold_bytes = 2 * (R * K + N * R + RL * K + N * RL) + 2 * lay_l["rank"] * (K + N)
    res["int4_lora_folded"] = {
        "workload": f"INT4 g64, rank {R} + LoRA rank {RL} folded (rank {lay_l['rank']}), "
                    "M 4608 x K 12288 -> N 3072",
        "timing": "back-to-back loop averages",
        "linear_us": round(t_lin_l * 1e6, 2),
        "linear_without_lora_us": round(t_lin_p * 1e6, 2),
        "fold_us": round(t_fold * 1e6, 2),
        "fold_timing": "per Python call, including its two output allocations (host-bound)",
        "fold_bytes": fold_bytes,
    }
    del x, lay, y, ws, codes, scales, lr, lay_l, ws_l, at, bt
    torch.cuda.empty_cache()

    # AWQ W4A16
    K, N = 3072, 12288
    aw = synth.WORKLOADS["awq"]
    w = torch.from_numpy(synth.gaussian((N, K), 0.02, 0, aw, 1)).to(dev)
    base = svdq.awq_quantize_weights(w)
    del w
    wbytes = N * K // 2 + 2 * N * (K // 64) * 2
    copies = max(1, int(512e6 // wbytes) + 1)
    lays = [base] + [dict(base, q=base["q"].clone(), scales=base["scales"].clone(),
                          zeros=base["zeros"].clone()) for _ in range(copies - 1)]
    awq = {}
    for m in (1, 16, 4608):
        x = torch.from_numpy(synth.activations(m, K, 0, aw, 0)).to(dev).to(torch.bfloat16)
        y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
        nrot = copies if m <= 64 else 1
        fn = lambda i: svdq.awq_linear_w4a16(x, lays[i % nrot], Y=y)
        # back-to-back loop average (at the weight-streaming sizes each call
        # reads a different weight copy), after a warm-up loop
        t = time_loop(fn, steps, warmup=steps)
        t_call = time_calls(fn, steps)
        byts = wbytes + m * K * 2 + m * N * 2
        flops = 2.0 * m * N * K
        r = {"avg_us": round(t * 1e6, 2), "per_call_bracket_us": round(float(t_call.mean()) * 1e6, 2),
             "timing": "back-to-back loop average",
             "algorithmic_bytes": byts,
             "GB/s": round(byts / t / 1e9, 1),
             "frac_hbm": round(byts / t / 1e9 / PEAK_HBM_GBS, 4),
             "TFLOP/s": round(flops / t / 1e12, 2),
             "frac_bf16_peak": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
             "bound": "hbm" if m <= 64 else "mfma (bf16)",
             "weight_copies_rotated": nrot}
        awq[f"M{m}"] = r
    res["awq_w4a16"] = dict(workload="AWQ W4A16 INT4 g64, bf16 scales / zeros, K 3072 -> N 12288",
                            **awq)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer shards "
              "over tokens with no exchange, so N GPUs would each run this same benchmark.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from w4a4_quantized_diffusion_amd import svdq, synth

    M, K, N, R = 4096, 3072, 12288, 32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_mb:
        src = torch.ones(args.copy_mb << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    s = synth.layer(M, K, N, R, seed=0, workload="flagship")
    W = torch.from_numpy(s["w"]).to(dev)
    xs = [torch.from_numpy(s["x"]).to(dev).to(torch.bfloat16)]
    for i in range(1, args.nbuf):
        xs.append(torch.from_numpy(synth.activations(M, K, 0, synth.WORKLOADS["flagship"],
                                                     10 + i)).to(dev).to(torch.bfloat16))
    bias = torch.from_numpy(s["b"]).to(dev).to(torch.bfloat16)
    amax = svdq.svdq_act_absmax(xs[0])
    layer = svdq.svdq_quantize_weights(W, amax, R, "int4")
    del W
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(args.nbuf)]
    ws = torch.empty(svdq.svdq_workspace_bytes(M, K, R), dtype=torch.uint8, device=dev)
    codes, scales, lr = svdq.workspace_views(ws, M, K, R)

    def step(i):
        svdq.svdq_linear_w4a4(xs[i % args.nbuf], layer, bias, workspace=ws,
                              Y=ys[i % args.nbuf])

    # The timed steps replay HIP graphs of the library calls, as a model's
    # forward pass would: one graph holds nbuf consecutive layer calls (each
    # on its own X / Y buffer), smaller ones the remainders of W and K modulo
    # nbuf, so exactly W and K steps run.  Warmup replays come right before the timed ones:
    # the GPU lowers its clock after a few ms idle and takes some tens of ms
    # of load to raise it again.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(args.nbuf):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(i)
        return g

    graphs = {n: capture(n) for n in {args.nbuf, args.steps % args.nbuf, args.warmup % args.nbuf}
              if n}

    def run_steps(k):
        for _ in range(k // args.nbuf):
            graphs[args.nbuf].replay()
        if k % args.nbuf:
            graphs[k % args.nbuf].replay()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    run_steps(args.steps)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps

    # eager: one library call per step from Python, for reference
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / args.steps

    # per-kernel durations, HIP events on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        x = xs[i % args.nbuf]
        evs[i][0].record()
        svdq.svdq_act_quantize(x, layer, codes, scales, lr)
        evs[i][1].record()
        svdq.svdq_gemm_w4a4(codes, scales, lr, layer, bias, Y=ys[i % args.nbuf])
        evs[i][2].record()
    torch.cuda.synchronize()
    t_act = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    t_gemm = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    t_gemm_loop = time_loop(lambda i: svdq.svdq_gemm_w4a4(codes, scales, lr, layer, bias,
                                                           Y=ys[i % args.nbuf]), args.steps)
    t_act_loop = time_loop(lambda i: svdq.svdq_act_quantize(xs[i % args.nbuf], layer, codes,
                                                            scales, lr), args.steps)

    ops = 2.0 * M * N * K
    value = ops / (ms_step * 1e-3) / 1e12
    gemm_tops = ops / t_gemm_loop / 1e12
    act_bytes = M * K * 2 + M * K // 2 + M * (K // 64) * 4 + M * R * 2 + K * 4 + R * K * 2
    gemm_bytes = (M * K // 2 + M * (K // 64) * 4 + M * R * 2 + N * K // 2 + N * (K // 64) * 4
                  + N * R * 2 + N * 2 + M * N * 2)
    traffic = traffic_from_profile(1)
    out = {
        "metric": "SVDQ W4A4 linear TOPS & % MFMA peak at M=4096,K=3072,N=12288,r=32",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": "SVDQuant W4A4 linear, INT4 g64, rank 32, M 4096 x K 3072 -> "
                               "N 12288, bf16 activations / bias / output",
                   "M": M, "K": K, "N": N, "rank": R, "precision": "int4-g64",
                   "parallelism": "none (1 GPU)"},
        "pct_of_mfma_peak": round(100.0 * value / PEAK_FP8_TOPS, 2),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 5),
        "eager_ms_per_step": round(ms_eager, 5),
        "timing": f"HIP graphs of {args.nbuf} consecutive layer calls replayed after the warmup "
                  "replays (eager per-call loop in eager_ms_per_step)",
        "roofline": {
            "kernel": "gemm_int4_kernel",
            "bound": "mfma",
            "achieved": round(gemm_tops, 2),
            "peak": PEAK_FP8_TOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tops / PEAK_FP8_TOPS, 4),
            "traffic": traffic,
            "algorithmic_ops_per_launch": ops,
            "algorithmic_bytes_per_launch": gemm_bytes,
            "avg_launch_us": round(t_gemm_loop * 1e6, 3),
        },
        "kernels": {
            "act_quant_int4": {"avg_us": round(t_act_loop * 1e6, 3),
                               "timing": "back-to-back loop average",
                               "per_call_bracket_us": round(float(t_act.mean()) * 1e6, 3),
                               "p95_per_call_bracket_us": round(float(np.percentile(t_act, 95)) * 1e6, 3),
                               "algorithmic_bytes": act_bytes,
                               "GB/s": round(act_bytes / t_act_loop / 1e9, 1),
                               "frac_hbm": round(act_bytes / t_act_loop / 1e9 / PEAK_HBM_GBS, 4)},
            "gemm_int4": {"avg_us": round(t_gemm_loop * 1e6, 3),
                          "timing": "back-to-back loop average",
                          "per_call_bracket_us": round(float(t_gemm.mean()) * 1e6, 3),
                          "p95_per_call_bracket_us": round(float(np.percentile(t_gemm, 95)) * 1e6, 3),
                          "TOPS": round(gemm_tops, 2)},
        },
        "gpu": torch.cuda.get_device_name(0),
    }
    del xs, ys, ws, layer, graphs
    torch.cuda.empty_cache()
    if not args.no_other_paths:
        out["other_paths"] = other_paths(args.other_steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(M, K, N, R, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
