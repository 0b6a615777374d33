"""SVDQuant W4A4 linear layer, INT4 precision: the oracle (test
infrastructure only; see the package docstring).

The method, as the pages state it in words (chaosnode.de page, "Die Technik:
SVDQuant"; aiphreaks.com page, "Technical Breakdown and Performance Metrics";
imaginepro.ai page, "Under the Hood"):

  1. outliers are moved out of the activations into the weights (per-channel
     smoothing),
  2. the hard part of the smoothed weight is kept as a 16-bit low-rank branch,
  3. the rest (the residual) and the smoothed activations are quantized to
     4 bits, and most of the compute runs on the 4-bit operands.

In symbols, with W [N, K] in nn.Linear layout and X [M, K]:

  lam_k    = sqrt(amax_x[k] / amax_w[k])        (migration strength 1/2)
  smooth_k = 1 / lam_k,  Xh = X * smooth,  Wh = W * lam
  Wh^T ~= L1h @ L2     (rank-r truncated SVD, L1h = U_r S_r, L2 = V_r^T)
  lora_down = (L1h / lam)^T  [r, K] bf16,  lora_up = L2^T  [N, r] bf16
  R = Wh - lam * (lora_up @ lora_down)
  Y = Q4(Xh) @ Q4(R)^T + bf16(X @ lora_down^T) @ lora_up^T + b

Q4 is symmetric INT4 in groups of 64 along K: scale = absmax / 7 (fp32),
code = round-half-even(z / scale) in [-7, 7].  Codes are stored as
sign-magnitude nibbles (bit 3 = sign, bits 0..2 = |code|; zero is 0x0), two
per byte, the even-k code in the low nibble.  Scales are fp32.

Floating-point steps the method rounds are written with fl32 / bf16; all other
arithmetic is float64.  The integer group products are exact (NumPy float32
matmul of integers whose partial sums stay below 2^24 is exact).
"""

import numpy as np

from .formats import fl32, bf16, bf16_bits, rne_int

F64 = np.float64
GROUP = 64


# --------------------------------------------------------------------------
# step 1: smoothing (outlier migration)
# --------------------------------------------------------------------------

def act_absmax(x):
    """Per-channel calibration statistic max_m |X[m, k]| (fp32, exact)."""
    return np.max(np.abs(np.asarray(x, dtype=np.float32)), axis=0)


def smoothing(act_amax, w):
    """lam and smooth = 1/lam per input channel.

    lam_k = fl32(sqrt(fl32(amax_x / amax_w))); lam_k = 1 where either
    statistic is zero.  smooth_k = fl32(1 / lam_k).  Returns (lam, smooth),
    both float32 [K]."""
    ax = np.asarray(act_amax, dtype=np.float32).astype(F64)
    aw = np.max(np.abs(np.asarray(w, dtype=np.float32)), axis=0).astype(F64)
    ok = (ax > 0) & (aw > 0)
    ratio = fl32(np.where(ok, ax / np.where(ok, aw, 1.0), 1.0)).astype(F64)
    lam = np.where(ok, fl32(np.sqrt(ratio)), np.float32(1.0)).astype(np.float32)
    smooth = fl32(1.0 / lam.astype(F64))
    return lam, smooth


# --------------------------------------------------------------------------
# step 2: truncated SVD of the smoothed weight, folded and rounded to bf16
# --------------------------------------------------------------------------

def truncated_svd(wh, rank):
    """Top-`rank` factors of Wh^T (K x N): L1h = U_r diag(S_r) [K, r],
    L2 = V_r^T [r, N], and all singular values.  Sign convention: the entry
    of largest magnitude of each left singular vector is positive (lowest
    index on ties)."""
    wh = np.asarray(wh, dtype=F64)
    u, s, vt = np.linalg.svd(wh.T, full_matrices=False)
    u, vt = u[:, :rank].copy(), vt[:rank, :].copy()
    for i in range(rank):
        j = int(np.argmax(np.abs(u[:, i])))
        if u[j, i] < 0:
            u[:, i] = -u[:, i]
            vt[i, :] = -vt[i, :]
    return u * s[:rank], vt, s


def fold_lowrank(l1h, l2, lam):
    """lora_down[i, k] = bf16(fl32(L1h[k, i] / lam_k)) and
    lora_up[n, i] = bf16(fl32(L2[i, n])); returned as float64 values."""
    lam = np.asarray(lam, dtype=np.float32).astype(F64)
    down = bf16(fl32(np.asarray(l1h, dtype=F64).T / lam[None, :]))
    up = bf16(fl32(np.asarray(l2, dtype=F64).T))
    return down, up


def residual(w, lam, lora_down, lora_up):
    """R[n, k] = fl32(W[n,k] lam_k - lam_k * sum_i lora_up[n,i] lora_down[i,k]),
    float64 arithmetic, the product Wh = W * lam exact."""
    lam = np.asarray(lam, dtype=np.float32).astype(F64)
    wh = np.asarray(w, dtype=np.float32).astype(F64) * lam[None, :]
    s = np.asarray(lora_up, dtype=F64) @ np.asarray(lora_down, dtype=F64)
    return fl32(wh - lam[None, :] * s)


# --------------------------------------------------------------------------
# step 3: symmetric INT4 group quantizer and nibble packing
# --------------------------------------------------------------------------

def quantize_int4(z):
    """Symmetric INT4, groups of 64 along the last axis.

    For each group: a = max|z|, s = fl32(a / 7); s == 0 gives all-zero codes,
    otherwise q = clamp(rne(fl32(z / s)), -8, 7).  Returns (q int8 [rows, K],
    s float32 [rows, K/64])."""
    z = np.asarray(z, dtype=np.float32)
    rows, k = z.shape
    assert k % GROUP == 0
    zg = z.reshape(rows, k // GROUP, GROUP).astype(F64)
    a = np.max(np.abs(zg), axis=2)
    s = fl32(a / 7.0)
    sd = s.astype(F64)[:, :, None]
    t = fl32(zg / np.where(sd > 0, sd, 1.0)).astype(F64)
    q = np.where(sd > 0, np.clip(rne_int(t), -8, 7), 0.0)
    return q.reshape(rows, k).astype(np.int8), s


def int4_to_nibble(q):
    """Signed code -> sign-magnitude nibble (zero is 0x0)."""
    q = np.asarray(q, dtype=np.int16)
    return np.where(q < 0, 8 | (-q), q).astype(np.uint8)


def nibble_to_int4(n):
    n = np.asarray(n, dtype=np.uint8)
    mag = (n & 7).astype(np.int8)
    return np.where(n & 8, -mag, mag).astype(np.int8)


def pack_nibbles(nib):
    """[rows, K] nibbles -> [rows, K/2] bytes; even k in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    out = np.empty((rows, 2 * half), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def pack_int4(q):
    return pack_nibbles(int4_to_nibble(q))


def unpack_int4(packed):
    return nibble_to_int4(unpack_nibbles(packed))


# --------------------------------------------------------------------------
# offline: weights -> quantized layer
# --------------------------------------------------------------------------

def quantize_weights(w, act_amax, rank, lowrank=None):
    """The offline half of the layer.

    w: [N, K] float32; act_amax: [K] float32 calibration max|X| (None: lam=1).
    lowrank: optional (lora_down, lora_up) float64 bf16-valued factors to use
    instead of computing the SVD (the SVD is not unique; this lets the later
    steps be compared for a given low-rank split).

    Returns a dict with smooth, lam, lora_down [r,K], lora_up [N,r] (float64
    bf16 values), R [N,K] float32, q (int8 codes) and sW [N, K/64] float32,
    wcodes [N, K/2] packed bytes, and the singular values."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if act_amax is None:
        lam = np.ones(k, dtype=np.float32)
        smooth = np.ones(k, dtype=np.float32)
    else:
        lam, smooth = smoothing(act_amax, w)
    sv = None
    if lowrank is not None:
        down, up = lowrank
        down = np.asarray(down, dtype=F64)
        up = np.asarray(up, dtype=F64)
    elif rank > 0:
        wh = w.astype(F64) * lam.astype(F64)[None, :]
        l1h, l2, sv = truncated_svd(wh, rank)
        down, up = fold_lowrank(l1h, l2, lam)
    else:
        down = np.zeros((0, k), dtype=F64)
        up = np.zeros((n, 0), dtype=F64)
    r = residual(w, lam, down, up)
    q, sw = quantize_int4(r)
    return dict(lam=lam, smooth=smooth, lora_down=down, lora_up=up, R=r,
                q=q, sW=sw, wcodes=pack_int4(q), sv=sv)


# --------------------------------------------------------------------------
# runtime: the activation side and the forward
# --------------------------------------------------------------------------

def smooth_activations(x, smooth):
    """Xh = fl32(X * smooth_k) (one fp32 multiply)."""
    x = np.asarray(x, dtype=np.float32).astype(F64)
    return fl32(x * np.asarray(smooth, dtype=np.float32).astype(F64)[None, :])


def quantize_activations(x, smooth):
    """The runtime activation step: (codes int8, sA float32) = Q4(Xh)."""
    return quantize_int4(smooth_activations(x, smooth))


def lowrank_down(x, lora_down):
    """LR[m, i] = bf16(fl32(sum_k bf16(X[m,k]) lora_down[i,k])), the sum in
    float64 (products of two bf16 values are exact there)."""
    xb = bf16(np.asarray(x, dtype=np.float32))
    return bf16(fl32(xb @ np.asarray(lora_down, dtype=F64).T))


def group_int_products(qx, qw, g):
    """I_g[m, n] = sum over k in group g of qx[m,k] qw[n,k], exact."""
    a = np.asarray(qx[:, g * GROUP:(g + 1) * GROUP], dtype=np.float32)
    b = np.asarray(qw[:, g * GROUP:(g + 1) * GROUP], dtype=np.float32)
    return (a @ b.T).astype(np.int64)


def quantized_branch(qx, sa, qw, sw):
    """sum_g sA[m,g] sW[n,g] I_g[m,n] in float64."""
    m, k = qx.shape
    n = qw.shape[0]
    y = np.zeros((m, n), dtype=F64)
    for g in range(k // GROUP):
        i_g = group_int_products(qx, qw, g).astype(F64)
        y += (sa[:, g].astype(F64)[:, None] * sw[:, g].astype(F64)[None, :]) * i_g
    return y


def linear_w4a4(x, layer, bias=None, row_block=512):
    """Y = Q4(Xh) Q4(R)^T + LR lora_up^T + b, float64.

    x: [M, K] float32 values (bf16 inputs are passed as their float32
    values).  layer: dict from quantize_weights (or one with the same keys:
    smooth, lora_down, lora_up, q, sW).  Returns (Y float64, dict of the
    intermediate activation-side results: qx, sA, LR)."""
    x = np.asarray(x, dtype=np.float32)
    m = x.shape[0]
    n = layer["q"].shape[0]
    y = np.empty((m, n), dtype=F64)
    qx_all, sa_all, lr_all = [], [], []
    up = np.asarray(layer["lora_up"], dtype=F64)
    for r0 in range(0, m, row_block):
        xb = x[r0:r0 + row_block]
        qx, sa = quantize_activations(xb, layer["smooth"])
        lr = lowrank_down(xb, layer["lora_down"])
        yb = quantized_branch(qx, sa, layer["q"], layer["sW"])
        yb += lr @ up.T
        if bias is not None:
            yb += np.asarray(bias, dtype=F64)[None, :]
        y[r0:r0 + row_block] = yb
        qx_all.append(qx)
        sa_all.append(sa)
        lr_all.append(lr)
    return y, dict(qx=np.concatenate(qx_all), sA=np.concatenate(sa_all),
                   LR=np.concatenate(lr_all))


def output_f32(y):
    return fl32(y)


def output_bf16_bits(y):
    return bf16_bits(fl32(y))


# ---------------------------------------------------------------- GELU input

def gelu_tanh(x):
    """GELU in its tanh form, the feed-forward activation between the MLP up-
    and down-projections (the original engine fuses it into its MLP kernels:
    chaosnode.de page, "Nunchaku Lite vs. Original"), in float64:
    0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, dtype=F64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def gelu_input(x):
    """The down-projection's input with GELU fused into the activation step:
    X' = bf16(gelu(X)) for bf16 X, the value an unfused GELU would store (fp32
    evaluation, then bf16).  Returns float32 values that are bf16 values."""
    return bf16(gelu_tanh(x)).astype(np.float32)



# ---------------------------------------------------------------- LoRA fold

def fold_lora(lora_down, lora_up, a, b, scale=1.0):
    """A LoRA adapter scale * B A (A [r_lora, K], B [N, r_lora], bf16 values)
    folded into the 16-bit low-rank branch by rank concatenation (LoRA loading
    keeps working on the quantized models: aiphreaks.com page, "Bringing
    Nunchaku 4-bit Diffusion Inference to Diffusers", Broader Ecosystem
    Impact).
    The branch reads raw X, as the adapter does, so

      lora_down' = [lora_down ; A ; 0],  lora_up' = [lora_up | bf16(fl32(scale B)) | 0]

    with the rank padded by zero rows / columns to a multiple of 16.  Returns
    (lora_down', lora_up', r_new) as float64 values."""
    a = np.asarray(a, dtype=F64)
    b = np.asarray(b, dtype=F64)
    r_lora, k = a.shape
    n = b.shape[0]
    down = np.zeros((0, k)) if lora_down is None else np.asarray(lora_down, dtype=F64)
    up = np.zeros((n, 0)) if lora_up is None else np.asarray(lora_up, dtype=F64)
    rank = down.shape[0]
    r_new = -(-(rank + r_lora) // 16) * 16
    pad = r_new - rank - r_lora
    bs = bf16(fl32(np.float32(scale) * b.astype(np.float32).astype(F64)))
    down2 = np.concatenate([down, a, np.zeros((pad, k))], axis=0)
    up2 = np.concatenate([up, bs, np.zeros((n, pad))], axis=1)
    return down2, up2, r_new
