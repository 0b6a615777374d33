"""Pins of the INT4 SVDQuant oracle against closed forms, invariants, special
cases that reduce to a library routine, and brute force on tiny inputs."""

import os

import numpy as np
import pytest

from oracle import svdq, formats as F
from w4a4_quantized_diffusion_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- smoothing

def test_smoothing_closed_form():
    w = np.zeros((3, 4), dtype=np.float32)
    w[0] = [0.5, 1.0, 0.25, 2.0]
    w[1] = [-0.25, 0.0, 0.0, 0.0]
    ax = np.array([2.0, 16.0, 0.0, 8.0], dtype=np.float32)
    lam, smooth = svdq.smoothing(ax, w)
    # sqrt(2/0.5) = 2, sqrt(16/1) = 4, zero statistic -> 1, sqrt(8/2) = 2
    assert list(lam) == [2.0, 4.0, 1.0, 2.0]
    assert list(smooth) == [0.5, 0.25, 1.0, 0.5]


def test_smoothing_rounds_in_fp32():
    w = np.array([[3.0]], dtype=np.float32)
    lam, smooth = svdq.smoothing(np.array([1.0], dtype=np.float32), w)
    assert lam[0] == np.float32(np.sqrt(np.float32(1.0 / 3.0)))
    assert smooth[0] == np.float32(1.0 / np.float64(lam[0]))


# ------------------------------------------------------------ INT4 quantizer

def _golden_group():
    rows = []
    with open(os.path.join(GOLDEN, "int4_group_ties.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append([float(t) for t in line.split()])
    return np.array(rows)


def test_int4_group_ties_golden():
    rows = _golden_group()
    z = np.zeros((1, 64), dtype=np.float32)
    z[0, :len(rows)] = rows[:, 0]
    q, s = svdq.quantize_int4(z)
    assert s[0, 0] == 2.0
    assert list(q[0, :len(rows)]) == list(rows[:, 1].astype(int))
    assert np.all(q[0, len(rows):] == 0)


def test_int4_error_bound_random():
    g = np.random.default_rng(5)
    z = (g.standard_normal((64, 512)) * np.exp(g.normal(0, 3, (64, 1)))).astype(np.float32)
    z[:, 7] *= 40
    q, s = svdq.quantize_int4(z)
    sd = np.repeat(s.astype(np.float64), 64, axis=1)
    err = np.abs(z.astype(np.float64) - sd * q)
    assert np.all(err <= 0.5 * sd * (1 + 2.0 ** -22))
    assert np.all(np.abs(q) <= 7)
    # the absmax element of every group maps to +-7
    zg = np.abs(z.reshape(64, 8, 64))
    qg = np.abs(q.reshape(64, 8, 64))
    assert np.all(np.take_along_axis(qg, np.argmax(zg, axis=2)[:, :, None], 2) == 7)


def test_int4_on_grid_is_lossless():
    g = np.random.default_rng(6)
    q0 = g.integers(-7, 8, size=(16, 256)).astype(np.int8)
    q0[:, ::64] = 7                                     # every group reaches 7
    e = g.integers(-20, 5, size=(16, 4))
    s0 = np.ldexp(1.0, e)
    z = (q0.reshape(16, 4, 64) * s0[:, :, None]).reshape(16, 256).astype(np.float32)
    q, s = svdq.quantize_int4(z)
    # s = fl32(7 * 2^e / 7) = 2^e exactly
    assert np.array_equal(s.astype(np.float64), s0)
    assert np.array_equal(q, q0)


def test_int4_symmetry_and_scaling():
    g = np.random.default_rng(7)
    z = g.standard_normal((8, 128)).astype(np.float32)
    q, s = svdq.quantize_int4(z)
    qn, sn = svdq.quantize_int4(-z)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for k in (-5, 3):
        qk, sk = svdq.quantize_int4(np.ldexp(z, k).astype(np.float32))
        assert np.array_equal(qk, q)
        assert np.array_equal(sk, np.ldexp(s, k).astype(np.float32))


def test_int4_zero_group():
    z = np.zeros((2, 128), dtype=np.float32)
    z[1, 64:] = 1.0
    q, s = svdq.quantize_int4(z)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert np.all(q[:, :64] == 0) and np.all(q[0] == 0) and np.all(q[1, 64:] == 7)


def test_nibble_packing_layout():
    q = np.array([[1, -2, 0, 7, -7, 3] + [0] * 58], dtype=np.int8)
    p = svdq.pack_int4(q)
    assert p.shape == (1, 32)
    # sign-magnitude: -2 -> 0xA, -7 -> 0xF; even k in the low nibble
    assert list(p[0, :3]) == [0xA1, 0x70, 0x3F]
    assert np.array_equal(svdq.unpack_int4(p), q)


# ------------------------------------------------------------------ SVD split

def _small_layer(seed=0, k=256, n=192, rank=8):
    g = np.random.default_rng(seed)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = g.standard_normal((32, k)).astype(np.float32)
    x[:, [3, 50, 77]] *= 30
    return x, w, rank


def test_svd_eckart_young_against_eigvalsh():
    x, w, r = _small_layer()
    lam, _ = svdq.smoothing(svdq.act_absmax(x), w)
    wh = w.astype(np.float64) * lam.astype(np.float64)[None, :]
    l1h, l2, _ = svdq.truncated_svd(wh, r)
    err = np.sum((wh.T - l1h @ l2) ** 2)
    ev = np.sort(np.linalg.eigvalsh(wh @ wh.T))[::-1]     # squared singular values
    assert err == pytest.approx(np.sum(ev[r:]), rel=1e-9)
    # no rank-r matrix does better: compare with a perturbed factorization
    assert np.sum((wh.T - (l1h + 1e-3) @ l2) ** 2) > err


def test_svd_factors_orthonormal_and_signed():
    x, w, r = _small_layer(1)
    wh = w.astype(np.float64)
    l1h, l2, s = svdq.truncated_svd(wh, r)
    u = l1h / s[:r][None, :]
    assert np.allclose(u.T @ u, np.eye(r), atol=1e-10)
    assert np.allclose(l2 @ l2.T, np.eye(r), atol=1e-10)
    j = np.argmax(np.abs(u), axis=0)
    assert np.all(u[j, np.arange(r)] > 0)


def test_residual_identity():
    x, w, r = _small_layer(2)
    layer = svdq.quantize_weights(w, svdq.act_absmax(x), r)
    lam = layer["lam"].astype(np.float64)
    wh = w.astype(np.float64) * lam[None, :]
    recon = lam[None, :] * (layer["lora_up"] @ layer["lora_down"]) + layer["R"].astype(np.float64)
    # Wh = diag(lam) L1 L2 + R up to the fp32 rounding of R
    ulp = np.spacing(np.abs(layer["R"])).astype(np.float64)
    assert np.all(np.abs(wh - recon) <= 0.5 * ulp * (1 + 1e-9) + 1e-300)
    # lora factors are bf16 values
    for t in (layer["lora_down"], layer["lora_up"]):
        assert np.array_equal(F.bf16(t), t)


def test_lowrank_absorbs_outliers():
    """With smoothing the outlier channels are heavy columns of Wh; the rank-r
    branch takes them, so the residual is much smaller than Wh there."""
    x, w, r = _small_layer(3)
    layer = svdq.quantize_weights(w, svdq.act_absmax(x), r)
    lam = layer["lam"]
    wh = w * lam[None, :]
    for c in (3, 50, 77):
        assert np.abs(layer["R"][:, c]).max() < 0.2 * np.abs(wh[:, c]).max()


# ------------------------------------------------------------------ forward

def _brute_force(x, layer, bias):
    """Triple loop over scalar Python floats on unpacked codes."""
    qx, sa = svdq.quantize_activations(x, layer["smooth"])
    lr = svdq.lowrank_down(x, layer["lora_down"])
    qw = svdq.unpack_int4(layer["wcodes"])
    m, k = x.shape
    n = qw.shape[0]
    y = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                g = kk // 64
                acc += float(sa[i, g]) * float(layer["sW"][j, g]) * int(qx[i, kk]) * int(qw[j, kk])
            for t in range(lr.shape[1]):
                acc += float(lr[i, t]) * float(layer["lora_up"][j, t])
            y[i, j] = acc + float(bias[j])
    return y


@pytest.mark.parametrize("k", [64, 128, 192])
def test_forward_brute_force_tiny(k):
    g = np.random.default_rng(k)
    m, n, r = 5, 7, 3
    w = (g.standard_normal((n, k)) * 0.05).astype(np.float32)
    x = g.standard_normal((m, k)).astype(np.float32)
    x[:, 1] *= 25
    b = (g.standard_normal(n) * 0.02).astype(np.float32)
    layer = svdq.quantize_weights(w, svdq.act_absmax(x), r)
    y, _ = svdq.linear_w4a4(x, layer, b)
    yb = _brute_force(x, layer, b)
    assert np.allclose(y, yb, rtol=1e-12, atol=1e-12)


def test_forward_on_grid_reduces_to_matmul():
    """lam = 1, rank 0, operands already on the INT4 grid with power-of-two
    scales: the layer is lossless and equals the float64 matmul X R^T."""
    g = np.random.default_rng(11)
    m, k, n = 9, 192, 13
    qa = g.integers(-7, 8, (m, k)); qa[:, ::64] = -7
    qb = g.integers(-7, 8, (n, k)); qb[:, 32::64] = 7
    ea = np.ldexp(1.0, g.integers(-6, 3, (m, k // 64)))
    eb = np.ldexp(1.0, g.integers(-9, -3, (n, k // 64)))
    x = (qa.reshape(m, 3, 64) * ea[:, :, None]).reshape(m, k).astype(np.float32)
    w = (qb.reshape(n, 3, 64) * eb[:, :, None]).reshape(n, k).astype(np.float32)
    layer = svdq.quantize_weights(w, None, 0)
    assert np.array_equal(layer["R"], w)
    b = g.standard_normal(n).astype(np.float32)
    y, aux = svdq.linear_w4a4(x, layer, b)
    assert np.array_equal(y, x.astype(np.float64) @ w.astype(np.float64).T + b)
    assert np.array_equal(aux["qx"], qa)


def test_forward_with_power_of_two_smoothing_is_exact():
    """Non-trivial smoothing pinned: calibration statistics chosen so that
    lam_k = 2^e_k exactly (e_k in -3..3), X = Xh_grid diag(lam) and
    W = Wh_grid diag(lam)^-1 with Xh_grid, Wh_grid on the INT4 grid (a code 7
    in every group, power-of-two group scales).  Smoothing must give back
    Xh_grid and Wh_grid exactly, so the layer is lossless: its codes are the
    grid codes and Y equals the float64 matmul X W^T + b.  Skipping the
    smoothing, or applying lam instead of 1/lam to X, moves X off the grid."""
    g = np.random.default_rng(13)
    m, k, n = 7, 192, 11
    qa = g.integers(-7, 8, (m, k)); qa[:, 5::64] = 7
    qb = g.integers(-7, 8, (n, k)); qb[:, 40::64] = -7
    ea = np.ldexp(1.0, g.integers(-5, 3, (m, k // 64)))
    eb = np.ldexp(1.0, g.integers(-8, -3, (n, k // 64)))
    e = g.integers(-3, 4, k)
    lam = np.ldexp(1.0, e)
    xh = (qa.reshape(m, 3, 64) * ea[:, :, None]).reshape(m, k)
    wh = (qb.reshape(n, 3, 64) * eb[:, :, None]).reshape(n, k)
    x = (xh * lam[None, :]).astype(np.float32)
    w = (wh / lam[None, :]).astype(np.float32)
    amax_w = np.max(np.abs(w), axis=0).astype(np.float32)
    amax_x = (amax_w.astype(np.float64) * np.ldexp(1.0, 2 * e)).astype(np.float32)
    l2, sm = svdq.smoothing(amax_x, w)
    assert np.array_equal(l2, lam.astype(np.float32)) and np.array_equal(sm, (1 / lam).astype(np.float32))
    layer = svdq.quantize_weights(w, amax_x, 0)
    assert np.array_equal(layer["R"], wh.astype(np.float32))
    assert np.array_equal(svdq.smooth_activations(x, layer["smooth"]), xh)
    b = g.standard_normal(n).astype(np.float32)
    y, aux = svdq.linear_w4a4(x, layer, b)
    assert np.array_equal(aux["qx"], qa)
    assert np.array_equal(y, x.astype(np.float64) @ w.astype(np.float64).T + b)
    # the same inputs without smoothing are off the grid: lossy
    y0, aux0 = svdq.linear_w4a4(x, dict(layer, smooth=np.ones(k, np.float32)), b)
    assert not np.array_equal(aux0["qx"], qa)


def test_forward_zero_residual_is_exact():
    """W exactly equal to a bf16 low-rank product (small integers): R == 0,
    every weight code is 0, and the layer returns X W^T + b exactly."""
    g = np.random.default_rng(12)
    m, k, n, r = 6, 128, 10, 4
    down = g.integers(-3, 4, (r, k)).astype(np.float64)
    up = g.integers(-3, 4, (n, r)).astype(np.float64)
    w = (up @ down).astype(np.float32)
    x = g.integers(-4, 5, (m, k)).astype(np.float32)
    layer = svdq.quantize_weights(w, None, r, lowrank=(down, up))
    assert np.all(layer["R"] == 0) and np.all(layer["wcodes"] == 0) and np.all(layer["sW"] == 0)
    b = g.integers(-2, 3, n).astype(np.float32)
    y, aux = svdq.linear_w4a4(x, layer, b)
    # |X lora_down^T| stays below 256, so the bf16 rounding of LR is exact
    assert np.abs(aux["LR"]).max() < 256
    assert np.array_equal(y, x.astype(np.float64) @ w.astype(np.float64).T + b)


def test_row_permutation_equivariance():
    s = synth.small()
    layer = svdq.quantize_weights(s["w"][:128, :256], svdq.act_absmax(s["x"][:, :256]), 4)
    x = s["x"][:, :256]
    y, _ = svdq.linear_w4a4(x, layer)
    p = np.random.default_rng(0).permutation(x.shape[0])
    yp, _ = svdq.linear_w4a4(x[p], layer)
    assert np.array_equal(yp, y[p])


def test_svdq_beats_naive_w4a4_on_small_workload():
    """Directional claim of the pages (imaginepro.ai "Under the Hood",
    chaosnode.de "Die Technik"): smoothing plus the low-rank branch gives
    a smaller error than plain W4A4.  Not a parity pin."""
    s = synth.small()
    x, w = s["x"], s["w"]
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    svd_layer = svdq.quantize_weights(w, svdq.act_absmax(x), s["rank"])
    naive = svdq.quantize_weights(w, None, 0)
    e_svd = np.sqrt(np.mean((svdq.linear_w4a4(x, svd_layer)[0] - exact) ** 2))
    e_naive = np.sqrt(np.mean((svdq.linear_w4a4(x, naive)[0] - exact) ** 2))
    assert e_svd < 0.5 * e_naive
