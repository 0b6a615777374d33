"""Seeded synthetic inputs shaped like the layers of a FLUX-class diffusion
transformer (the pages' workload: 1024x1024 images from FLUX.1 / ERNIE
checkpoints, which are not available here).

This module only draws numbers; it contains none of the layer's arithmetic.
Both the product path and the CPU oracle take their inputs from here.

Every draw uses numpy.random.default_rng([seed, workload_id, tensor_id]).
Activations are drawn in float32 and, where the workload is bf16, rounded to
bf16 (round-to-nearest-even) so both sides see exactly the same values.

Workloads (ids are fixed; shapes follow the diffusion-transformer layers):
  0 "small":    X fp32 64x1024 ~N(0,1), 8 outlier channels x30 (exact),
                W [1024,1024] ~N(0,0.02), b ~N(0,0.02), rank 16.
  1 "attn":     X bf16 4608x3072 (4096 image + 512 text tokens) ~N(0,1),
                1% of channels (31) scaled by U(20,50) per channel;
                QKV W [9216,3072], out W [3072,3072] ~N(0,0.02), rank 32.
  2 "mlp":      up W [12288,3072], down W [3072,12288]; M 4608 or 9216.
  3 "mlp_fp4":  the mlp shapes for the NVFP4 precision.
  4 "awq":      X bf16 M in {1,16,4608} x 3072, W [12288,3072].
  5 "flagship": X bf16 4096x3072, W [12288,3072], rank 32 (attn/mlp
                distributions).
"""

import numpy as np

WORKLOADS = {"small": 0, "attn": 1, "mlp": 2, "mlp_fp4": 3, "awq": 4, "flagship": 5, "lora": 6}


def rng(seed, workload, tensor):
    return np.random.default_rng([int(seed), int(workload), int(tensor)])


def round_bf16(x):
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def to_bf16_bits(x):
    """float32 values that are already bf16 values -> uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def gaussian(shape, std, seed, workload, tensor):
    g = rng(seed, workload, tensor)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def activations(m, k, seed, workload, tensor, n_outliers=None, lo=20.0, hi=50.0,
                fixed_factor=None, bf16=True):
    """X ~ N(0,1) [m, k] with heavy-tailed outlier channels.

    n_outliers channels (default 1% of k, rounded down) are chosen without
    replacement and scaled per channel by U(lo, hi), or by fixed_factor."""
    g = rng(seed, workload, tensor)
    x = g.standard_normal(size=(m, k), dtype=np.float32)
    if n_outliers is None:
        n_outliers = k // 100
    gc = rng(seed, workload, tensor + 1000)
    ch = gc.choice(k, size=n_outliers, replace=False)
    if fixed_factor is not None:
        f = np.full(n_outliers, fixed_factor, dtype=np.float32)
    else:
        f = gc.uniform(lo, hi, size=n_outliers).astype(np.float32)
    x[:, ch] *= f[None, :]
    return round_bf16(x) if bf16 else x


def small(seed=0):
    """Workload 0: the small single-layer case (fp32 activations)."""
    w = WORKLOADS["small"]
    x = activations(64, 1024, seed, w, 0, n_outliers=8, fixed_factor=30.0, bf16=False)
    return dict(x=x, w=gaussian((1024, 1024), 0.02, seed, w, 1),
                b=gaussian((1024,), 0.02, seed, w, 2), rank=16)


def layer(m, k, n, rank, seed=0, workload="flagship", bias=True, x_tensor=0):
    """A bf16-activation layer of the given shape (attn/mlp distributions).
    Weights depend only on (seed, workload, k, n), activations on (m, k)."""
    w = WORKLOADS[workload]
    wt = 10 + (k * 131 + n) % 997
    x = activations(m, k, seed, w, x_tensor)
    out = dict(x=x, w=gaussian((n, k), 0.02, seed, w, wt), rank=rank)
    out["b"] = round_bf16(gaussian((n,), 0.02, seed, w, wt + 1)) if bias else None
    return out


def calibration(m, k, seed=0, workload="flagship"):
    """Calibration activations drawn like the runtime ones (other tensor id)."""
    return activations(m, k, seed, WORKLOADS[workload], 0)


def random_bytes(shape, seed, workload, tensor):
    g = rng(seed, workload, tensor)
    return g.integers(0, 256, size=shape, dtype=np.uint8)


def random_int4_layer(n, k, rank, seed=0, workload="flagship"):
    """A quantized INT4 layer drawn directly (no SVD), for runtime tests and
    timing at full size.  Codes are uniform on -7..7 in the packed
    sign-magnitude nibble format (two per byte, even k low); weight scales,
    smoothing factors and low-rank factors are positive / Gaussian draws, the
    factors rounded to bf16.  Returns numpy arrays: wcodes u8 [n, k/2],
    sW f32 [n, k/64], smooth f32 [k], lora_down / lora_up bf16 bit patterns
    (uint16) [rank, k] / [n, rank]."""
    w = WORKLOADS[workload]
    g = rng(seed, w, 900)
    mag = g.integers(0, 8, size=(n, k), dtype=np.uint8)
    neg = (g.integers(0, 2, size=(n, k), dtype=np.uint8) == 1) & (mag != 0)
    nib = mag | (neg.astype(np.uint8) << 3)
    wcodes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    sw = (g.uniform(0.5, 2.0, size=(n, k // 64)) * 2e-3).astype(np.float32)
    smooth = g.uniform(0.05, 0.5, size=k).astype(np.float32)
    down = to_bf16_bits(round_bf16((g.standard_normal((rank, k)) * 0.05).astype(np.float32)))
    up = to_bf16_bits(round_bf16((g.standard_normal((n, rank)) * 0.02).astype(np.float32)))
    return dict(wcodes=wcodes, sW=sw, smooth=smooth, lora_down_bits=down, lora_up_bits=up)


def lora_adapter(n, k, r_lora, seed=0, std=0.05):
    """A LoRA adapter's factors A [r_lora, K] and B [N, r_lora]: Gaussian
    entries of the given std, rounded to bf16 values (float32)."""
    w = WORKLOADS["lora"]
    return (round_bf16(gaussian((r_lora, k), std, seed, w, 1)),
            round_bf16(gaussian((n, r_lora), std, seed, w, 2)))
