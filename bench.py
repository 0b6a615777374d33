#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 linear layer on one MI355X.

One step is one full layer call (svdq_linear_w4a4: the fused activation
kernel, then the W4xA4 GEMM with its low-rank / bias epilogue) on one batch
of seeded synthetic activations, inputs resident in HBM.  The timed steps
are library calls issued back to back from Python with a HIP event after
each one (per-step p50 / p95 from the differences); replays of one-step HIP
graphs of the same call are timed too and reported beside them.  Before the
timed steps the layer is replayed for a fixed wall time (--ramp-ms)
whatever --warmup is, because the GPU lowers its clock when idle and takes
tens of milliseconds of load to raise it again; the ramp's length is its own
field.

Workload: the FLUX-scale projection M 4096 x K 3072 -> N 12288, rank 32,
INT4 groups of 64, bf16 activations / bias / output.  Weights are quantized
once, offline, by the library's own svdq_quantize_weights.

Prints one JSON line: TOPS = 2 M N K / (time per step), the roofline of the
dominant kernel (the GEMM) measured with HIP events on the launch stream, and
the CPU oracle's throughput on a bounded sample of the same layer (the very
codes and scales the GPU used), with a same-run parity check of the GPU's
output rows.  "other_paths" holds the INT4 layer at the DiT projection shapes
(attention QKV / output at 4608 tokens, MLP up-projection at 4608 and 9216
tokens, the MLP down-projection with its GELU fused), the NVFP4 precision at
the MLP up-projection and the AWQ W4A16 layer at M = 1, 16, 4608.

  python bench.py [--steps K] [--warmup W] [--ramp-ms T] [--no-cpu-baseline]
                  [--no-other-paths]
"""

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_INT8_TOPS = 5000.0         # MI355X dense INT8 / FP8 MFMA
PEAK_FP6_TOPS = 10100.0         # dense FP6 / FP4 MFMA (the INT4 GEMM's instruction)
PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0        # dense fp16 / bf16 MFMA
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP4_TFLOPS = 10100.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--ramp-ms", type=float, default=200.0,
                    help="replay the layer for at least this wall time before timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-svd-timing", action="store_true",
                    help="skip timing the oracle's SVD of the flagship weight")
    ap.add_argument("--nbuf", type=int, default=4, help="distinct X / Y buffers rotated")
    ap.add_argument("--no-other-paths", action="store_true",
                    help="skip the other shapes, NVFP4 and AWQ W4A16")
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


def traffic_from_profile():
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


# ------------------------------------------------------------ environment

def _sclk_file():
    for d in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(d, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
        except OSError:
            continue
        p = os.path.join(d, "pp_dpm_sclk")
        if os.access(p, os.R_OK):
            return p
    return None


def read_sclk_mhz(path):
    """The active shader-clock level (the line marked '*'), MHz, or None."""
    try:
        with open(path) as f:
            for line in f:
                if "*" in line:
                    m = re.search(r"(\d+)\s*[Mm][Hh][Zz]", line)
                    if m:
                        return int(m.group(1))
    except OSError:
        pass
    return None


class ClockSampler:
    """Samples the active shader-clock level from sysfs every `period` s on a
    host thread (no GPU work) while the timed region runs."""

    def __init__(self, period=0.01):
        self.path = _sclk_file()
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._t = None

    def __enter__(self):
        if self.path:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def _run(self):
        while not self._stop.is_set():
            v = read_sclk_mhz(self.path)
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __exit__(self, *exc):
        self._stop.set()
        if self._t:
            self._t.join()

    def summary(self):
        if not self.path:
            return {"mhz_median": None, "note": "no readable pp_dpm_sclk in sysfs"}
        if not self.samples:
            return {"mhz_median": None, "note": f"{self.path} gave no active level"}
        s = sorted(self.samples)
        return {"mhz_median": s[len(s) // 2], "mhz_min": s[0], "mhz_max": s[-1],
                "samples": len(s), "source": self.path}


def rocm_versions():
    import torch
    v = {"torch": torch.__version__, "torch_hip": torch.version.hip}
    try:
        with open("/opt/rocm/.info/version") as f:
            v["rocm"] = f.read().strip()
    except OSError:
        v["rocm"] = None
    return v


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_info():
    try:
        from threadpoolctl import threadpool_info
        return [{k: i.get(k) for k in ("internal_api", "version", "num_threads",
                                       "threading_layer", "architecture")}
                for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # noqa: BLE001
        return []


# ------------------------------------------------------------ CPU oracle leg

def cpu_baseline(ctx, seconds, time_svd):
    """The oracle forward (INT4 quantization of the activations, exact group
    products, fp64 scaled accumulation, bf16 low-rank branch) on a bounded
    sample of rows of the same layer the GPU ran (its codes, scales and
    factors, read back), timed on the host cores; a 1-thread figure on a
    smaller sample; the oracle's SVD of the flagship weight on its own; and a
    same-run parity check: the GPU's activation codes and scales on every row
    bit-exact, its output rows of the sample within the layer's tolerance
    (max |dY| <= 1e-2 rms(Y) + 2^-8 |Y| for bf16 output)."""
    import numpy as np
    from oracle import svdq as O
    from oracle import formats as F
    from w4a4_quantized_diffusion_amd import layout
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # noqa: BLE001
        threadpool_limits = None
    M, K, N, R = ctx["M"], ctx["K"], ctx["N"], ctx["rank"]
    x = ctx["x"]
    lay = dict(q=O.unpack_int4(layout.int4_from_device(ctx["wcodes"])),
               sW=np.ascontiguousarray(ctx["wscales"].T), smooth=ctx["smooth"],
               lora_down=F.bf16_to_f32(ctx["lora_down_bits"]).astype(np.float64),
               lora_up=F.bf16_to_f32(ctx["lora_up_bits"]).astype(np.float64))
    bias = ctx["bias"]
    affinity = len(os.sched_getaffinity(0))
    blas = blas_info()
    threads = min([b["num_threads"] for b in blas if b.get("num_threads")] + [affinity])

    def grow(budget, rows=8):
        while True:                  # grow the sample until it is ~1/8 of the budget
            t0 = time.perf_counter()
            O.linear_w4a4(x[:rows], lay, bias)
            t = time.perf_counter() - t0
            if t > budget / 8 or rows >= M:
                break
            rows = min(M, rows * 2)
        return min(M, max(rows, int(rows * (budget / max(t, 1e-9)))))

    rows = grow(seconds)
    t0 = time.perf_counter()
    y_ref, inter = O.linear_w4a4(x[:rows], lay, bias)
    t = time.perf_counter() - t0
    tops = 2.0 * rows * N * K / t / 1e12
    out = {"value": tops, "unit": "TOPS", "cores": threads, "kind": "oracle",
           "sample": f"rows 0..{rows - 1} of {M} of the same layer (full K={K}, N={N}, "
                     f"rank {R}, bias), {t:.1f} s, numpy with {threads} BLAS threads",
           "cpu_model": cpu_model(), "affinity_cpus": affinity, "blas": blas}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            r1 = grow(seconds / 4, rows=4)
            t0 = time.perf_counter()
            O.linear_w4a4(x[:r1], lay, bias)
            t1 = time.perf_counter() - t0
        out["value_1thread"] = 2.0 * r1 * N * K / t1 / 1e12
        out["sample_1thread"] = f"rows 0..{r1 - 1}, {t1:.1f} s, 1 BLAS thread"
    if time_svd:
        lam, _ = O.smoothing(ctx["amax"], ctx["w"])
        wh = ctx["w"].astype(np.float64) * lam.astype(np.float64)[None, :]
        t0 = time.perf_counter()
        O.truncated_svd(wh, R)
        out["svd_seconds"] = round(time.perf_counter() - t0, 2)
        out["svd"] = (f"oracle truncated SVD (LAPACK full SVD, float64) of the smoothed "
                      f"{N}x{K} weight, {threads} BLAS threads")
    # same-run parity of the GPU's results
    qx, sa = O.quantize_activations(x, lay["smooth"])
    codes_ok = bool(np.array_equal(layout.int4_from_device(ctx["act_codes"]), O.pack_int4(qx)))
    scales_ok = bool(np.array_equal(np.ascontiguousarray(ctx["act_scales"].T), sa))
    yg = ctx["y"][:rows].astype(np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    tol = 1e-2 * rms + 2.0 ** -8 * np.abs(y_ref)
    err = np.abs(yg - y_ref)
    out["parity"] = {"act_codes_bit_exact_all_rows": codes_ok,
                     "act_scales_bit_exact_all_rows": scales_ok,
                     "y_rows_checked": rows,
                     "y_within_tolerance": bool(np.all(err <= tol)),
                     "y_max_err_over_rms": round(float(err.max()) / rms, 6),
                     "y_tolerance": "1e-2 rms(Y) + 2^-8 |Y| per element"}
    return out


# ------------------------------------------------------------ timing helpers

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


GRAPH_CALLS = 50   # consecutive calls captured in one graph by time_loop
KERNEL_CALLS = 200  # least number of launches behind each per-kernel average
TIMING_LOOP = f"HIP graph of {GRAPH_CALLS} consecutive calls, replayed; events around the replays"
TIMING_LOOPS = TIMING_LOOP.replace("graph of", "graphs of")

def time_eager(fn, steps, warmup=3):
    """Average duration (seconds) of fn(i) issued back to back from Python,
    HIP events on the current stream around the whole loop.  For kernels of
    a few microseconds the host's issue rate can be the limit: time_loop
    removes it."""
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


def time_loop(fn, steps, warmup=3):
    """Average duration (seconds) of fn(i) on the GPU: calls i = 0 .. n-1
    (n = min(steps, GRAPH_CALLS)) captured back to back in one HIP graph,
    replayed until at least `steps` calls have run, HIP events on the
    replay stream around the replays.  The calls and their inputs are the
    same as when issued eagerly; the graph only takes the host's issue time
    per call out of the measurement."""
    import math
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    n = max(1, min(steps, GRAPH_CALLS))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    for _ in range(max(1, warmup // n)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(steps / n))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) * 1e-3 / (reps * n)


def pct(a, q):
    import numpy as np
    return round(float(np.percentile(a, q)) * 1e6, 3)


def act_bytes_int4(M, K, R):
    """Algorithmic bytes of the INT4 activation kernel: X read (bf16), codes
    (4 bit) and scales (fp32 per 64) and LR (bf16) written, smooth and
    lora_down read once."""
    return M * K * 2 + M * K // 2 + M * (K // 64) * 4 + M * R * 2 + K * 4 + R * K * 2


def gemm_bytes_int4(M, K, N, R):
    """Algorithmic bytes of the INT4 GEMM: both code / scale sets, LR and
    lora_up read once, bias read, Y (bf16) written."""
    return (M * K // 2 + M * (K // 64) * 4 + M * R * 2 + N * K // 2 + N * (K // 64) * 4
            + N * R * 2 + N * 2 + M * N * 2)


# ------------------------------------------------------------ other paths

def int4_case(M, K, N, R, workload, steps, seed):
    """The INT4 layer at one DiT projection shape: weights quantized by the
    library from a seeded synthetic weight, the GPU time per call of the
    layer and of its two kernels (time_loop) after a warm-up of the same
    length."""
    import torch
    from w4a4_quantized_diffusion_amd import svdq, synth
    dev = torch.device("cuda:0")
    s = synth.layer(M, K, N, R, seed=seed, workload=workload)
    x = torch.from_numpy(s["x"]).to(dev).to(torch.bfloat16)
    bias = torch.from_numpy(s["b"]).to(dev).to(torch.bfloat16)
    lay = svdq.svdq_quantize_weights(torch.from_numpy(s["w"]).to(dev), svdq.svdq_act_absmax(x),
                                     R, "int4")
    del s
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(svdq.svdq_workspace_bytes(M, K, R), dtype=torch.uint8, device=dev)
    codes, scales, lr = svdq.workspace_views(ws, M, K, R)
    t_lin = time_loop(lambda i: svdq.svdq_linear_w4a4(x, lay, bias, workspace=ws, Y=y), steps,
                      warmup=steps)
    t_act = time_loop(lambda i: svdq.svdq_act_quantize(x, lay, codes, scales, lr), steps,
                      warmup=steps)
    t_gem = time_loop(lambda i: svdq.svdq_gemm_w4a4(codes, scales, lr, lay, bias, Y=y), steps,
                      warmup=steps)
    ops = 2.0 * M * N * K
    ab = act_bytes_int4(M, K, R)
    return {"workload": f"INT4 g64, rank {R}, M {M} x K {K} -> N {N}, bf16 in / bias / out",
            "timing": TIMING_LOOPS,
            "linear_us": round(t_lin * 1e6, 2),
            "TOPS": round(ops / t_lin / 1e12, 1),
            "pct_of_int8_peak": round(100.0 * ops / t_lin / 1e12 / PEAK_INT8_TOPS, 2),
            "gemm_int4_us": round(t_gem * 1e6, 2),
            "gemm_TOPS": round(ops / t_gem / 1e12, 1),
            "gemm_frac_int8_peak": round(ops / t_gem / 1e12 / PEAK_INT8_TOPS, 4),
            "gemm_frac_fp6_peak": round(ops / t_gem / 1e12 / PEAK_FP6_TOPS, 4),
            "act_quant_int4_us": round(t_act * 1e6, 2),
            "act_quant_frac_hbm": round(ab / t_act / 1e9 / PEAK_HBM_GBS, 4)}


def other_paths(steps):
    """The INT4 layer at the DiT projection shapes (attention QKV / output at
    M 4608, MLP up-projection at M 4608 and 9216), the NVFP4 precision at the
    MLP up-projection shape (M 4608, K 3072 -> N 12288, rank 32), the INT4
    MLP down-projection with the GELU fused in (M 4608, K 12288 -> N 3072),
    the same layer with a LoRA adapter folded in, and the AWQ W4A16 layer
    (K 3072 -> N 12288) at M = 1, 16 and 4608: seeded synthetic tensors,
    weights quantized by the library (the down-projection's INT4 layer drawn
    directly), per-kernel HIP-event times.  Weight-streaming cases rotate
    enough weight copies (> 512 MB) that the 256 MB last-level cache cannot
    hold them."""
    import numpy as np
    import torch
    from w4a4_quantized_diffusion_amd import svdq, synth, layout
    dev = torch.device("cuda:0")
    res = {}

    for name, (M, K, N, wl) in {"int4_attn_qkv": (4608, 3072, 9216, "attn"),
                                "int4_attn_out": (4608, 3072, 3072, "attn"),
                                "int4_mlp_up": (4608, 3072, 12288, "mlp"),
                                "int4_mlp_up_batch2": (9216, 3072, 12288, "mlp")}.items():
        res[name] = int4_case(M, K, N, 32, wl, steps, seed=3)
        torch.cuda.empty_cache()

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
        "timing": TIMING_LOOPS,
        "gemm_nvfp4": {"avg_us": round(t_gem_loop * 1e6, 2),
                       "per_call_bracket_us": round(float(t_gem.mean()) * 1e6, 2),
                       "TFLOP/s": round(ops / t_gem_loop / 1e12, 1), "bound": "mfma (f16)",
                       "frac_f16_peak": round(ops / t_gem_loop / 1e12 / PEAK_F16_TFLOPS, 4),
                       "frac_fp4_peak": round(ops / t_gem_loop / 1e12 / PEAK_FP4_TFLOPS, 4)},
        "act_quant_nvfp4": {"avg_us": round(t_act_loop * 1e6, 2),
                            "per_call_bracket_us": round(float(t_act.mean()) * 1e6, 2),
                            "timing": TIMING_LOOP,
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
    act_bytes = act_bytes_int4(M, K, R)
    res["int4_mlp_down_gelu"] = {
        "workload": "INT4 g64, rank 32, GELU fused into the activation pass, "
                    "M 4608 x K 12288 -> N 3072",
        "timing": TIMING_LOOPS,
        "linear_us": round(t_lin_g * 1e6, 2),
        "TOPS": round(ops / t_lin_g / 1e12, 1),
        "pct_of_int8_peak": round(100.0 * ops / t_lin_g / 1e12 / PEAK_INT8_TOPS, 2),
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
    t_fold = time_eager(lambda i: svdq.svdq_fold_lora(lay, at, bt, 1.0), 20, warmup=5)
    t_lin_l = time_loop(lambda i: svdq.svdq_linear_w4a4(x, lay_l, workspace=ws_l, Y=y), steps,
                        warmup=steps)
    fold_bytes = 2 * (R * K + N * R + RL * K + N * RL) + 2 * lay_l["rank"] * (K + N)
    res["int4_lora_folded"] = {
        "workload": f"INT4 g64, rank {R} + LoRA rank {RL} folded (rank {lay_l['rank']}), "
                    "M 4608 x K 12288 -> N 3072",
        "timing": TIMING_LOOPS,
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
        # GPU time per call (at the weight-streaming sizes each call reads a
        # different weight copy), after a warm-up of the same length
        t = time_loop(fn, steps, warmup=steps)
        t_call = time_calls(fn, steps)
        byts = wbytes + m * K * 2 + m * N * 2
        flops = 2.0 * m * N * K
        r = {"avg_us": round(t * 1e6, 2), "per_call_bracket_us": round(float(t_call.mean()) * 1e6, 2),
             "timing": TIMING_LOOP,
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


# ------------------------------------------------------------ the flagship

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
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    layer = svdq.svdq_quantize_weights(W, amax, R, "int4")
    torch.cuda.synchronize()
    t_quant = time.perf_counter() - t0
    del W
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(args.nbuf)]
    ws = torch.empty(svdq.svdq_workspace_bytes(M, K, R), dtype=torch.uint8, device=dev)
    codes, scales, lr = svdq.workspace_views(ws, M, K, R)

    def step(i):
        svdq.svdq_linear_w4a4(xs[i % args.nbuf], layer, bias, workspace=ws,
                              Y=ys[i % args.nbuf])

    # One-step HIP graphs of the library call, one per X / Y buffer: they
    # ramp the clock, and their replay rate is reported beside the timed calls.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(args.nbuf):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(args.nbuf):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)

    # clock ramp: replay for a fixed wall time, then the requested warmup steps
    t0 = time.perf_counter()
    n_ramp = 0
    while True:
        for _ in range(16):
            graphs[n_ramp % args.nbuf].replay()
            n_ramp += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= args.ramp_ms:
            break
    ramp_ms = (time.perf_counter() - t0) * 1e3
    for i in range(args.warmup):
        step(i)

    # timed: K library calls issued back to back, a HIP event after each
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(args.steps):
            step(i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_step = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]) * 1e-3

    # the same steps as one-step HIP graph replays, for reference
    for i in range(args.warmup):
        graphs[i % args.nbuf].replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        graphs[i % args.nbuf].replay()
    e1.record()
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / args.steps

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
    # the per-kernel averages run at least KERNEL_CALLS launches whatever K
    # is (a single graph replay of 20 launches varies by several percent)
    kn = max(args.steps, KERNEL_CALLS)
    t_gemm_loop = time_loop(lambda i: svdq.svdq_gemm_w4a4(codes, scales, lr, layer, bias,
                                                           Y=ys[i % args.nbuf]), kn, warmup=kn)
    t_act_loop = time_loop(lambda i: svdq.svdq_act_quantize(xs[i % args.nbuf], layer, codes,
                                                            scales, lr), kn, warmup=kn)
    t_gemm_eager = time_eager(lambda i: svdq.svdq_gemm_w4a4(codes, scales, lr, layer, bias,
                                                            Y=ys[i % args.nbuf]), kn)
    t_act_eager = time_eager(lambda i: svdq.svdq_act_quantize(xs[i % args.nbuf], layer, codes,
                                                              scales, lr), kn)

    ops = 2.0 * M * N * K
    value = ops / (ms_step * 1e-3) / 1e12
    gemm_tops = ops / t_gemm_loop / 1e12
    act_bytes = act_bytes_int4(M, K, R)
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
        "pct_of_mfma_peak": round(100.0 * value / PEAK_INT8_TOPS, 2),
        "peak_note": "MFMA peak = MI355X dense INT8 5.0 POPS (the GEMM runs on FP6 MFMAs, "
                     "dense peak 10.1 PFLOP/s: roofline.frac_instruction)",
        "step_p50_us": pct(per_step, 50),
        "step_p95_us": pct(per_step, 95),
        "step_timing": f"library calls issued back to back, a HIP event after each; {args.nbuf} "
                       "X / Y buffers rotated",
        "clock_ramp_ms": round(ramp_ms, 1),
        "clock_ramp_replays": n_ramp,
        "wall_ms_per_step": round(wall / args.steps * 1e3, 5),
        "graph_ms_per_step": round(ms_graph, 5),
        "sclk_during_timed_steps": clk.summary(),
        "roofline": {
            "kernel": "gemm_int4_kernel",
            "bound": "mfma",
            "achieved": round(gemm_tops, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
            "traffic": traffic_from_profile(),
            "peak_instruction": PEAK_FP6_TOPS,
            "frac_instruction": round(gemm_tops / PEAK_FP6_TOPS, 4),
            "instruction": "v_mfma_scale_f32_32x32x64_f8f6f4, FP6-E2M3 operands",
            "algorithmic_ops_per_launch": ops,
            "algorithmic_bytes_per_launch": gemm_bytes_int4(M, K, N, R),
            "avg_launch_us": round(t_gemm_loop * 1e6, 3),
            "gemm_source_sha": gemm_source_sha(),
        },
        "kernels": {
            "act_quant_int4": {"avg_us": round(t_act_loop * 1e6, 3),
                               "timing": TIMING_LOOP,
                               "eager_loop_us": round(t_act_eager * 1e6, 3),
                               "per_call_bracket_p50_us": pct(t_act, 50),
                               "per_call_bracket_p95_us": pct(t_act, 95),
                               "algorithmic_bytes": act_bytes,
                               "GB/s": round(act_bytes / t_act_loop / 1e9, 1),
                               "frac_hbm": round(act_bytes / t_act_loop / 1e9 / PEAK_HBM_GBS, 4)},
            "gemm_int4": {"avg_us": round(t_gemm_loop * 1e6, 3),
                          "timing": TIMING_LOOP,
                          "eager_loop_us": round(t_gemm_eager * 1e6, 3),
                          "per_call_bracket_p50_us": pct(t_gemm, 50),
                          "per_call_bracket_p95_us": pct(t_gemm, 95),
                          "TOPS": round(gemm_tops, 2)},
        },
        "offline_quantize_weights_s": round(t_quant, 3),
        "gpu": torch.cuda.get_device_name(0),
        "gpu_arch": torch.cuda.get_device_properties(0).gcnArchName,
        "versions": rocm_versions(),
    }
    ctx = None
    if not args.no_cpu_baseline:
        # what the oracle leg needs, read back before the device buffers go
        svdq.svdq_act_quantize(xs[0], layer, codes, scales, lr)
        svdq.svdq_linear_w4a4(xs[0], layer, bias, workspace=ws, Y=ys[0])
        torch.cuda.synchronize()
        ctx = {"M": M, "K": K, "N": N, "rank": R, "w": s["w"], "amax": amax.cpu().numpy(),
               "x": xs[0].float().cpu().numpy(), "bias": bias.double().cpu().numpy(),
               "y": ys[0].float().cpu().numpy(),
               "act_codes": codes.cpu().numpy(), "act_scales": scales.cpu().numpy(),
               "wcodes": layer["wcodes"].cpu().numpy(), "wscales": layer["wscales"].cpu().numpy(),
               "smooth": layer["smooth"].cpu().numpy(),
               "lora_down_bits": layer["lora_down"].cpu().numpy().view(np.uint16),
               "lora_up_bits": layer["lora_up"].cpu().numpy().view(np.uint16)}
    del xs, ys, ws, layer, graphs, codes, scales, lr
    torch.cuda.empty_cache()
    if not args.no_other_paths:
        out["other_paths"] = other_paths(args.other_steps)
    if ctx is not None:
        out["cpu_baseline"] = cpu_baseline(ctx, args.cpu_seconds, not args.no_svd_timing)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
