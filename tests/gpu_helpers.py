"""Shared helpers of the GPU parity tests: move oracle results and seeded
inputs to the device, and compare with the documented tolerances."""

import numpy as np
import torch

from oracle import formats as F
from oracle import svdq as O
from w4a4_quantized_diffusion_amd import synth


def dev():
    return torch.device("cuda:0")


def t_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def t_bf16_bits(values):
    """float values (already bf16-representable or not) -> int16 tensor of
    their RNE bf16 bit patterns."""
    bits = F.bf16_bits(np.asarray(values, dtype=np.float64))
    return torch.from_numpy(bits.view(np.int16).copy()).to(dev())


def t_x(x, bf16):
    """Activations to the device: bf16 tensor (values must be bf16) or fp32."""
    t = t_f32(x)
    if bf16:
        t2 = t.to(torch.bfloat16)
        assert torch.equal(t2.float(), t), "activation values are not bf16 values"
        return t2
    return t


def t_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def gm_codes(packed):
    """Row-major packed codes [rows, K/2] -> group-major [K/64, rows, 32]."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    return np.ascontiguousarray(packed.reshape(rows, half // 32, 32).transpose(1, 0, 2))


def rm_codes(gm):
    """Group-major [K/64, rows, 32] -> row-major [rows, K/2]."""
    gm = np.asarray(gm, dtype=np.uint8)
    g, rows, _ = gm.shape
    return np.ascontiguousarray(gm.transpose(1, 0, 2).reshape(rows, g * 32))


# INT4 device codes ("fold" format, from its definition in include/svdq.h):
# chunk c of a row's 32 bytes per group holds k = 8c + j as field j and
# k = 32 + 8c + j as field 8 + j; field f (|q| in bits 0..2, sign in bit 5)
# sits at bits 6f.. of a 96-bit string o0 | o1 << 32 | o2 << 64, stored as
# X = o0 | (o1 & GX), Y = o2 | (o1 & GY).  Written here with explicit bit
# arrays, independently of the package's converter.
_GX, _GY = 0x18618618, 0x61861861
_W32 = (np.uint64(1) << np.arange(32, dtype=np.uint64))


def _chunk_codes(q):
    """q [rows, K] -> [K/64, rows, 4 chunks, 16 fields] codes."""
    rows, k = q.shape
    g = k // 64
    out = np.empty((g, rows, 4, 16), dtype=np.int64)
    for c in range(4):
        for j in range(8):
            out[:, :, c, j] = q[:, 8 * c + j::64].T
            out[:, :, c, 8 + j] = q[:, 32 + 8 * c + j::64].T
    return out


def gm_int4(packed):
    """Oracle INT4 codes (textbook sign-magnitude nibbles [rows, K/2]) ->
    device fold format [K/64, rows, 32] bytes."""
    q = O.unpack_int4(np.asarray(packed, dtype=np.uint8)).astype(np.int64)
    cq = _chunk_codes(q)
    pat = np.abs(cq) | ((cq < 0).astype(np.int64) << 5)         # 6-bit fields
    bits = ((pat[..., None] >> np.arange(6)) & 1).reshape(cq.shape[:-1] + (96,))
    words = (bits.reshape(bits.shape[:-1] + (3, 32)).astype(np.uint64) * _W32).sum(-1)
    o0, o1, o2 = words[..., 0], words[..., 1], words[..., 2]
    x = o0 | (o1 & np.uint64(_GX))
    y = o2 | (o1 & np.uint64(_GY))
    xy = np.stack([x, y], axis=-1).astype("<u4")                # [g, rows, 4, 2]
    return np.ascontiguousarray(xy.view(np.uint8).reshape(q.shape[1] // 64, q.shape[0], 32))


def rm_int4(dev):
    """Device fold-format codes [K/64, rows, 32] -> textbook nibbles
    [rows, K/2], keeping the sign bit of a zero magnitude (so a negative zero
    shows as 0x8 and fails a comparison with the oracle's codes)."""
    dev = np.ascontiguousarray(np.asarray(dev, dtype=np.uint8))
    g, rows, _ = dev.shape
    w = dev.view("<u4").reshape(g, rows, 4, 2).astype(np.uint64)
    x, y = w[..., 0], w[..., 1]
    o0 = x & np.uint64(~_GX & 0xFFFFFFFF)
    o1 = (x & np.uint64(_GX)) | (y & np.uint64(_GY))
    o2 = y & np.uint64(~_GY & 0xFFFFFFFF)
    words = np.stack([o0, o1, o2], axis=-1)                     # [g, rows, 4, 3]
    bits = ((words[..., None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).astype(np.int64)
    fb = bits.reshape(g, rows, 4, 16, 6)
    nib = fb[..., 0] | (fb[..., 1] << 1) | (fb[..., 2] << 2) | (fb[..., 5] << 3)
    out = np.empty((rows, g * 64), dtype=np.uint8)
    for c in range(4):
        for j in range(8):
            out[:, 8 * c + j::64] = nib[:, :, c, j].T
            out[:, 32 + 8 * c + j::64] = nib[:, :, c, 8 + j].T
    return (out[:, 0::2] | (out[:, 1::2] << 4)).astype(np.uint8)


def gm_scales(s):
    return np.ascontiguousarray(np.asarray(s).T)


def layer_to_device(lay, rank, n, k, prec=0):
    """An oracle INT4 layer dict -> the binding's device layer dict."""
    d = dict(rank=rank, prec=prec, N=n, K=k)
    d["smooth"] = t_f32(lay["smooth"])
    d["lora_down"] = t_bf16_bits(lay["lora_down"]) if rank else torch.zeros(1, dtype=torch.int16, device=dev())
    d["lora_up"] = t_bf16_bits(lay["lora_up"]) if rank else torch.zeros(1, dtype=torch.int16, device=dev())
    d["wcodes"] = t_u8(gm_int4(lay["wcodes"]))
    d["wscales"] = t_f32(gm_scales(lay["sW"]))
    d["w_tensor_scale"] = torch.ones(1, dtype=torch.float32, device=dev())
    d["x_tensor_scale"] = torch.ones(1, dtype=torch.float32, device=dev())
    return d


def random_int4_layer(n, k, rank, seed, workload="flagship"):
    """The seeded synthetic layer of synth.random_int4_layer in the oracle's
    dict form (codes unpacked, factors as float64 values)."""
    r = synth.random_int4_layer(n, k, rank, seed, workload)
    return dict(q=O.unpack_int4(r["wcodes"]), sW=r["sW"], wcodes=r["wcodes"],
                smooth=r["smooth"], lora_down=F.bf16_to_f32(r["lora_down_bits"]).astype(np.float64),
                lora_up=F.bf16_to_f32(r["lora_up_bits"]).astype(np.float64))


def bf16_bits_np(t):
    return t.cpu().numpy().view(np.uint16) if t.dtype == torch.int16 else \
        t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_ulp_diff(a_bits, b_bits):
    """Distance in representable steps between two bf16 bit arrays."""
    def key(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(key(a_bits) - key(b_bits))


def assert_lr_close(lr_gpu, x, down, what=""):
    """LR = bf16(sum_k bf16(X) lora_down) accumulated in fp32 on the GPU:
    |LR_gpu - exact| <= 2^-8 |exact| (bf16 rounding, which may go either way
    from a slightly different fp32 sum) + 2 K 2^-24 sum_k |x_k d_k| (a bound
    on the fp32 summation error in any order).  Where the dot product
    cancels this is wider than one bf16 step.  Returns the count of entries
    that are not the oracle's bits."""
    xb = F.bf16(np.asarray(x, dtype=np.float32))
    d = np.asarray(down, dtype=np.float64)
    exact = xb @ d.T
    sabs = np.abs(xb) @ np.abs(d).T
    k = xb.shape[1]
    got = F.bf16_to_f32(bf16_bits_np(lr_gpu)).astype(np.float64)
    tol = 2.0 ** -8 * np.abs(exact) + 2.0 * k * 2.0 ** -24 * sabs
    err = np.abs(got - exact)
    assert np.all(err <= tol), f"{what}: LR out of tolerance at {np.argwhere(err > tol)[:5]}"
    ref_bits = F.bf16_bits(F.fl32(exact))
    return int((bf16_bits_np(lr_gpu) != ref_bits).sum())


def y_tolerance(y_ref, bf16_out):
    """max|dY| <= 1e-2 rms(Y); bf16 output adds 2^-8 |Y| per element (the
    output rounding alone)."""
    rms = np.sqrt(np.mean(y_ref ** 2))
    tol = 1e-2 * rms
    if bf16_out:
        tol = tol + 2.0 ** -8 * np.abs(y_ref)
    return tol


def assert_y_close(y_gpu, y_ref, bf16_out, what=""):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    tol = y_tolerance(y_ref, bf16_out)
    err = np.abs(y - y_ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance; "
                           f"max err {err.max():.3e}, rms(Y) {np.sqrt(np.mean(y_ref ** 2)):.3e}")
    return float(err.max() / np.sqrt(np.mean(y_ref ** 2)))


def degenerate_activations(seed=0, k=256, m=24):
    """fp32 activations that hit the quantizers' special cases: an all-zero
    row, all-zero / constant / subnormal / huge (1e30) groups, one outlier in
    a group of zeros, groups of equal magnitudes, and rows scaled by 10^e for
    e in [-40, 30] (scales that underflow to zero or become subnormal)."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((m, k)).astype(np.float32)
    x[0] = 0
    x[1, 0:64] = 0
    x[1, 64:128] = 3.0
    x[1, 128:192] = (g.choice([-1, 1], 64) * 1e-42).astype(np.float32)
    x[1, 192:256] = (g.standard_normal(64) * 1e30).astype(np.float32)
    x[2] = 0
    for b in range(k // 16):
        x[2, 16 * b + (b * 5) % 16] = 5.0 if b % 2 else -5.0
    x[3] = np.where(g.integers(0, 2, k) == 1, 2.5, -2.5).astype(np.float32)
    for r in range(4, m):
        x[r] *= np.float32(10.0 ** g.uniform(-40, 30))
    return x
