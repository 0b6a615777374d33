"""NVFP4-style precision of the SVDQuant W4A4 layer: the oracle (test
infrastructure only; see the package docstring).

The pages name NVFP4 as the svdq_w4a4 precision for Blackwell GPUs
(aiphreaks.com page, "Technical Breakdown"; chaosnode.de page,
"Hardware-Support"; the French announcement names an "nvfp4_r32"
checkpoint).  They give no recipe; the reading used here is the common NVFP4
layout:

* values are FP4 E2M1 in blocks of 16 along K,
* each block has an FP8 E4M3 scale,
* each tensor has one fp32 scale ts = amax / (6 * 448) (1 when amax is 0).

Per block of 16 values z of a tensor with scale ts:
  a   = max |z|
  sb  = E4M3_rne_sat(fl32(a / fl32(6 ts)))
  den = fl32(decode(sb) * ts)
  e   = E2M1_rne_sat(fl32(z / den))   (all zero when den == 0)
and the dequantized value is decode(e) * decode(sb) * ts.

Weights use ts_w from max|R|; activations use a static ts_x from the
calibration statistic: ts_x = fl32(max_k fl32(amax_x[k] smooth_k) / 2688).
Smoothing, the low-rank branch and the residual are those of the INT4
precision (module svdq).
"""

import numpy as np

from .formats import fl32, e4m3_encode, e4m3_decode, e2m1_encode, e2m1_decode
from . import svdq

F64 = np.float64
BLOCK = 16
FP4_MAX_TIMES_E4M3_MAX = 6.0 * 448.0      # 2688


def tensor_scale(amax):
    """fl32(amax / 2688), or 1 when amax is 0."""
    amax = float(amax)
    return np.float32(1.0) if amax == 0.0 else fl32(amax / FP4_MAX_TIMES_E4M3_MAX)[()]


def quantize_nvfp4(z, ts):
    """Blocks of 16 along the last axis.  Returns (codes uint8 [rows, K]
    nibbles, block scales uint8 [rows, K/16] E4M3 codes)."""
    z = np.asarray(z, dtype=np.float32)
    rows, k = z.shape
    assert k % BLOCK == 0
    zb = z.reshape(rows, k // BLOCK, BLOCK).astype(F64)
    a = np.max(np.abs(zb), axis=2)
    d = fl32(6.0 * np.float64(ts)).astype(F64)
    sb = e4m3_encode(fl32(a / d))
    den = fl32(e4m3_decode(sb) * np.float64(ts)).astype(F64)[:, :, None]
    t = fl32(zb / np.where(den > 0, den, 1.0))
    e = np.where(den > 0, e2m1_encode(t), 0).astype(np.uint8)
    return e.reshape(rows, k), sb


def dequantize_nvfp4(codes, sb, ts):
    rows, k = codes.shape
    v = e2m1_decode(codes).reshape(rows, k // BLOCK, BLOCK)
    return (v * e4m3_decode(sb)[:, :, None] * np.float64(ts)).reshape(rows, k)


def quantize_weights(w, act_amax, rank, lowrank=None):
    """Offline half, NVFP4 precision.  Same smoothing / SVD / residual as the
    INT4 precision; R is quantized with blocks of 16 and an fp32 tensor scale.
    Also returns the static activation tensor scale ts_x."""
    base = svdq.quantize_weights(w, act_amax, rank, lowrank=lowrank)
    r = base["R"]
    ts_w = tensor_scale(np.max(np.abs(r.astype(F64))) if r.size else 0.0)
    codes, sbw = quantize_nvfp4(r, ts_w)
    if act_amax is None:
        ts_x = np.float32(1.0)
    else:
        xs = fl32(np.asarray(act_amax, dtype=np.float32).astype(F64)
                  * base["smooth"].astype(F64))
        ts_x = tensor_scale(np.max(xs))
    out = dict(base)
    del out["q"], out["sW"]
    out.update(codes=codes, sbw=sbw, ts_w=np.float32(ts_w), ts_x=np.float32(ts_x),
               wcodes=svdq.pack_nibbles(codes))
    return out


def quantize_activations(x, smooth, ts_x):
    return quantize_nvfp4(svdq.smooth_activations(x, smooth), ts_x)


def linear_nvfp4(x, layer, bias=None, row_block=512):
    """Y = ts_x ts_w sum_b sbx sbw P_b + LR lora_up^T + b in float64, with
    P_b the exact block dot products of the E2M1 values."""
    x = np.asarray(x, dtype=np.float32)
    m = x.shape[0]
    n = layer["codes"].shape[0]
    wd = dequantize_nvfp4(layer["codes"], layer["sbw"], 1.0)     # without ts_w
    up = np.asarray(layer["lora_up"], dtype=F64)
    ts = np.float64(layer["ts_x"]) * np.float64(layer["ts_w"])
    y = np.empty((m, n), dtype=F64)
    ex_all, sbx_all, lr_all = [], [], []
    for r0 in range(0, m, row_block):
        xb = x[r0:r0 + row_block]
        ex, sbx = quantize_activations(xb, layer["smooth"], layer["ts_x"])
        xd = dequantize_nvfp4(ex, sbx, 1.0)
        lr = svdq.lowrank_down(xb, layer["lora_down"])
        yb = ts * (xd @ wd.T) + lr @ up.T
        if bias is not None:
            yb += np.asarray(bias, dtype=F64)[None, :]
        y[r0:r0 + row_block] = yb
        ex_all.append(ex)
        sbx_all.append(sbx)
        lr_all.append(lr)
    return y, dict(codes=np.concatenate(ex_all), sbx=np.concatenate(sbx_all),
                   LR=np.concatenate(lr_all))
