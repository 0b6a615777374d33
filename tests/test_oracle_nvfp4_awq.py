"""Pins of the NVFP4 and AWQ W4A16 oracles: closed forms, lossless on-grid
cases that reduce to a float64 matmul, error bounds and special cases."""

import numpy as np
import pytest

from oracle import nvfp4, awq, svdq, formats as F


# ------------------------------------------------------------------ NVFP4

def test_tensor_scale_closed_form():
    assert nvfp4.tensor_scale(2688.0) == 1.0
    assert nvfp4.tensor_scale(0.0) == 1.0
    assert nvfp4.tensor_scale(5376.0) == 2.0
    assert nvfp4.tensor_scale(1.0) == np.float32(1.0 / 2688.0)


def test_nvfp4_on_grid_is_lossless():
    """Blocks built as e * sb with max|e| = 6 and E4M3 sb, tensor scale 1:
    the quantizer returns the same codes and block scales."""
    g = np.random.default_rng(21)
    rows, k = 8, 128
    codes = g.integers(0, 16, (rows, k)).astype(np.uint8)
    codes[codes == 8] = 0
    codes[:, ::16] = 7                                   # |e| = 6 in every block
    sb = g.integers(1, 0x7E, (rows, k // 16)).astype(np.uint8)
    sb[0, 0] = 0x7E                                      # 448: global amax 2688
    z = nvfp4.dequantize_nvfp4(codes, sb, 1.0).astype(np.float32)
    ts = nvfp4.tensor_scale(np.abs(z.astype(np.float64)).max())
    assert ts == 1.0
    c2, sb2 = nvfp4.quantize_nvfp4(z, ts)
    assert np.array_equal(c2, codes) and np.array_equal(sb2, sb)


def test_nvfp4_error_bound_and_range():
    g = np.random.default_rng(22)
    z = (g.standard_normal((32, 256)) * 0.3).astype(np.float32)
    z[:, 5] *= 40
    ts = nvfp4.tensor_scale(np.abs(z).max())
    codes, sb = nvfp4.quantize_nvfp4(z, ts)
    den = F.fl32(F.e4m3_decode(sb) * np.float64(ts)).astype(np.float64)
    den = np.repeat(den, 16, axis=1)
    t = z.astype(np.float64) / den
    dec = F.e2m1_decode(codes)
    # inside the grid the error is at most half the local grid step
    grid = F.E2M1_POS
    step = np.interp(np.abs(dec), grid[:-1], np.diff(grid))
    inside = np.abs(t) <= 6
    assert np.all(np.abs(t - dec)[inside] <= 0.5 * np.maximum(step, 1.0)[inside] + 1e-6)
    assert np.all(np.abs(dec) <= 6)
    assert np.all(F.e4m3_decode(sb) <= 448)


def test_nvfp4_zero_tensor():
    c, sb = nvfp4.quantize_nvfp4(np.zeros((2, 32), np.float32), nvfp4.tensor_scale(0.0))
    assert np.all(c == 0) and np.all(sb == 0)


def test_nvfp4_forward_on_grid_reduces_to_matmul():
    g = np.random.default_rng(23)
    m, k, n = 5, 64, 6
    cx = g.integers(0, 16, (m, k)).astype(np.uint8); cx[cx == 8] = 0; cx[:, ::16] = 7
    cw = g.integers(0, 16, (n, k)).astype(np.uint8); cw[cw == 8] = 0; cw[:, 3::16] = 15
    sx = g.integers(0x30, 0x50, (m, k // 16)).astype(np.uint8); sx[0, 0] = 0x7E
    sw = g.integers(0x30, 0x50, (n, k // 16)).astype(np.uint8); sw[0, 0] = 0x7E
    x = nvfp4.dequantize_nvfp4(cx, sx, 1.0).astype(np.float32)
    w = nvfp4.dequantize_nvfp4(cw, sw, 1.0).astype(np.float32)
    layer = nvfp4.quantize_weights(w, None, 0)
    assert layer["ts_w"] == 1.0 and np.array_equal(layer["codes"], cw)
    layer["ts_x"] = np.float32(1.0)
    y, aux = nvfp4.linear_nvfp4(x, layer)
    assert np.array_equal(aux["codes"], cx) and np.array_equal(aux["sbx"], sx)
    assert np.array_equal(y, x.astype(np.float64) @ w.astype(np.float64).T)


def test_nvfp4_activation_tensor_scale_static():
    g = np.random.default_rng(24)
    x = g.standard_normal((16, 64)).astype(np.float32)
    w = (g.standard_normal((8, 64)) * 0.02).astype(np.float32)
    amax = svdq.act_absmax(x)
    layer = nvfp4.quantize_weights(w, amax, 2)
    xs = np.max(F.fl32(amax.astype(np.float64) * layer["smooth"].astype(np.float64)))
    assert layer["ts_x"] == F.fl32(np.float64(xs) / 2688.0)


# -------------------------------------------------------------------- AWQ

def test_awq_on_grid_is_lossless():
    g = np.random.default_rng(31)
    n, k = 6, 128
    q0 = g.integers(0, 16, (n, k)).astype(np.uint8)
    q0[:, ::64] = 0
    q0[:, 1::64] = 15
    z0 = g.integers(0, 16, (n, k // 64)).astype(np.float64)
    s0 = F.bf16(np.ldexp(g.uniform(1, 2, (n, k // 64)), g.integers(-10, -4, (n, k // 64))))
    # exact multiples of s0 that keep mx - mn = 15 s0 exactly representable
    w = ((q0.reshape(n, 2, 64) - z0[:, :, None]) * s0[:, :, None]).reshape(n, k).astype(np.float32)
    q, s, z, packed = awq.quantize_weights(w)
    assert np.array_equal(s, s0) and np.array_equal(z, z0) and np.array_equal(q, q0)
    # power-of-two scales: (q - z) s has at most 4 significant bits, so the
    # 16-bit weights are the weights themselves and Y is the exact product
    s2 = np.ldexp(1.0, g.integers(-10, -4, (n, k // 64)))
    w2 = ((q0.reshape(n, 2, 64) - z0[:, :, None]) * s2[:, :, None]).reshape(n, k).astype(np.float32)
    q2, s2q, z2, _ = awq.quantize_weights(w2)
    x = g.standard_normal((4, k)).astype(np.float32)
    y = awq.linear_w4a16(x, q2, s2q, z2)
    assert np.allclose(y, x.astype(np.float64) @ w2.astype(np.float64).T, rtol=0, atol=1e-12)


def test_awq_bf16_weight_rounding_bound():
    """The 16-bit weights differ from the exact dequantized ones by at most
    half a bf16 step (2^-8 relative: 8 significant bits), so
    |Y - X wd_exact^T| <= 2^-8 sum|x||wd|;
    and they are bf16 values."""
    g = np.random.default_rng(34)
    w = (g.standard_normal((24, 192)) * 0.05).astype(np.float32)
    q, s, z, _ = awq.quantize_weights(w)
    wd = awq.dequantize(q, s, z)
    wb = awq.dequantize_bf16(q, s, z)
    assert np.array_equal(F.bf16(wb), wb)
    assert np.all(np.abs(wb - wd) <= 2.0 ** -8 * np.abs(wd))
    assert np.any(wb != wd)                  # 12-bit products do get rounded
    x = g.standard_normal((5, 192)).astype(np.float32)
    y = awq.linear_w4a16(x, q, s, z)
    exact = x.astype(np.float64) @ wd.T
    assert np.all(np.abs(y - exact) <= 2.0 ** -8 * (np.abs(x) @ np.abs(wd).T) + 1e-12)


def test_awq_zero_points_are_positive_zero():
    w = np.zeros((1, 128), np.float32)
    w[0, :64] = np.linspace(0.0, 1.0, 64)        # min 0: zero point 0
    _, s, z, _ = awq.quantize_weights(w)
    assert z[0, 0] == 0 and not np.signbit(z[0, 0])
    assert z[0, 1] == 0 and not np.signbit(z[0, 1]) and s[0, 1] == 0


def test_awq_error_bound():
    g = np.random.default_rng(32)
    w = (g.standard_normal((16, 256)) * 0.02).astype(np.float32)
    q, s, z, _ = awq.quantize_weights(w)
    wd = awq.dequantize(q, s, z)
    sd = np.repeat(s, 64, axis=1)
    # bf16 scale rounding can push the top code past 15 by a fraction of a step
    assert np.all(np.abs(w - wd) <= 0.5 * sd * (1 + 2 ** -7) + 2 * sd * (q == 15) + 2 * sd * (q == 0))
    assert np.median(np.abs(w - wd) / sd) < 0.3
    assert q.max() <= 15 and z.max() <= 15


def test_awq_zero_group_and_all_positive():
    w = np.zeros((2, 64), np.float32)
    w[1] = np.linspace(0.1, 1.5, 64)
    q, s, z, _ = awq.quantize_weights(w)
    assert s[0, 0] == 0 and z[0, 0] == 0 and np.all(q[0] == 0)
    # min clamped to 0: zero point 0, top value maps to 15
    assert z[1, 0] == 0 and q[1, -1] == 15


def test_awq_packing_roundtrip():
    g = np.random.default_rng(33)
    w = g.standard_normal((3, 128)).astype(np.float32)
    q, s, z, packed = awq.quantize_weights(w)
    assert np.array_equal(awq.unpack(packed), q)
    assert packed.shape == (3, 64)
