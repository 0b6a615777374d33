"""Pins of the oracle's LoRA fold (an adapter scale * B A carried by the
16-bit low-rank branch through a longer rank) against facts that do not
depend on its own formula: an integer layer whose folded output is the exact
matmul with W + scale B A; the adapter's exact contribution scale X A^T B^T
within the bf16 rounding bound; scale 0 and the zero padding leaving the
layer unchanged; and two folds in a row agreeing with one fold of the
concatenated adapters."""

import numpy as np
import pytest

from oracle import svdq as O
from oracle import formats as F


def _base(seed, k=192, n=48, rank=16, m=20):
    g = np.random.default_rng(seed)
    w = (g.standard_normal((n, k)) * 0.05).astype(np.float32)
    x = F.bf16(g.standard_normal((m, k)).astype(np.float32)).astype(np.float32)
    x[:, 7] *= 16
    layer = O.quantize_weights(w, O.act_absmax(x), rank)
    return g, x, layer


def _with(layer, down, up):
    out = dict(layer)
    out.update(lora_down=down, lora_up=up)
    return out


def test_fold_integer_layer_is_exact_matmul():
    """R == 0 (W a product of small integers), an integer adapter and
    scale 1/2: every rounding is exact and Y = X (W + B A / 2)^T + b."""
    g = np.random.default_rng(3)
    m, k, n, r, rl = 7, 128, 12, 16, 5
    down = g.integers(-3, 4, (r, k)).astype(np.float64)
    up = g.integers(-3, 4, (n, r)).astype(np.float64)
    w = (up @ down).astype(np.float32)
    layer = O.quantize_weights(w, None, r, lowrank=(down, up))
    assert np.all(layer["R"] == 0)
    a = g.integers(-2, 3, (rl, k)).astype(np.float64)
    b = g.integers(-4, 5, (n, rl)).astype(np.float64)
    d2, u2, r_new = O.fold_lora(layer["lora_down"], layer["lora_up"], a, b, 0.5)
    assert r_new == 32 and d2.shape == (32, k) and u2.shape == (n, 32)
    x = g.integers(-2, 3, (m, k)).astype(np.float32)
    bias = g.integers(-2, 3, n).astype(np.float32)
    y, aux = O.linear_w4a4(x, _with(layer, d2, u2), bias)
    assert np.abs(aux["LR"]).max() < 256          # bf16 LR exact
    ref = x.astype(np.float64) @ (w.astype(np.float64) + 0.5 * (b @ a)).T + bias
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("rank,rl,scale", [(16, 16, 1.0), (32, 5, 0.7), (0, 9, -1.3)])
def test_fold_adds_the_adapter_within_bf16(rank, rl, scale):
    """Y_folded - Y_base against the adapter's exact contribution
    scale (X A^T) B^T: only the bf16 rounding of X A^T and of scale B (2^-8
    relative each) separates them."""
    g, x, layer = _base(rank + rl, rank=rank)
    k, n = x.shape[1], layer["q"].shape[0]
    a = F.bf16(g.standard_normal((rl, k)) * 0.05)
    b = F.bf16(g.standard_normal((n, rl)) * 0.05)
    d2, u2, r_new = O.fold_lora(layer["lora_down"] if rank else None,
                                layer["lora_up"] if rank else None, a, b, scale)
    assert r_new == -(-(rank + rl) // 16) * 16
    y0, _ = O.linear_w4a4(x, layer)
    y1, _ = O.linear_w4a4(x, _with(layer, d2, u2))
    xa = x.astype(np.float64) @ a.T
    exact = scale * xa @ b.T
    bound = (2.0 ** -7 + 2.0 ** -16) * (np.abs(xa) @ np.abs(scale * b).T) + 1e-12
    assert np.all(np.abs((y1 - y0) - exact) <= bound)
    # the bound is not vacuous: the contribution is far above it
    assert np.abs(exact).max() > 20 * bound.max()


def test_fold_zero_scale_and_padding_leave_layer():
    g, x, layer = _base(5)
    k, n = x.shape[1], layer["q"].shape[0]
    a = F.bf16(g.standard_normal((3, k)))
    b = F.bf16(g.standard_normal((n, 3)))
    d2, u2, r_new = O.fold_lora(layer["lora_down"], layer["lora_up"], a, b, 0.0)
    assert r_new == 32
    assert np.array_equal(d2[:16], layer["lora_down"]) and np.array_equal(d2[16:19], a)
    assert np.all(d2[19:] == 0) and np.all(u2[:, 16:] == 0)
    assert np.array_equal(u2[:, :16], layer["lora_up"])
    y0, _ = O.linear_w4a4(x, layer)
    y1, _ = O.linear_w4a4(x, _with(layer, d2, u2))
    assert np.allclose(y1, y0, rtol=1e-13, atol=1e-13)


def test_two_folds_equal_one_concatenated_fold():
    g, x, layer = _base(6)
    k, n = x.shape[1], layer["q"].shape[0]
    a1, a2 = F.bf16(g.standard_normal((16, k))), F.bf16(g.standard_normal((16, k)))
    b1, b2 = F.bf16(g.standard_normal((n, 16))), F.bf16(g.standard_normal((n, 16)))
    d, u, r1 = O.fold_lora(layer["lora_down"], layer["lora_up"], a1, b1, 0.25)
    d, u, r2 = O.fold_lora(d, u, a2, b2, 0.25)
    dc, uc, rc = O.fold_lora(layer["lora_down"], layer["lora_up"], np.concatenate([a1, a2]),
                             np.concatenate([b1, b2], axis=1), 0.25)
    assert (r1, r2, rc) == (32, 48, 48)
    assert np.array_equal(d, dc) and np.array_equal(u, uc)
