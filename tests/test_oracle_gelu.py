"""Pins of the oracle's GELU (the fused input form of the MLP
down-projection) against facts that do not depend on its own formula: the
exact erf form, which the tanh form approximates to within 4.8e-4; the
odd-part identity gelu(x) - gelu(-x) = x; the limits 0 and x far out; and
bf16 rounding of the fused input."""

import math

import numpy as np

from oracle import svdq as O
from oracle import formats as F


def test_gelu_tanh_close_to_erf_form():
    x = np.linspace(-8.0, 8.0, 40001)
    erf_form = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    d = np.abs(O.gelu_tanh(x) - erf_form)
    assert d.max() <= 4.8e-4
    # the approximation is not exact anywhere but the origin region
    assert d[np.abs(x) > 0.5].max() > 1e-5


def test_gelu_odd_part_is_identity():
    x = np.random.default_rng(0).normal(0.0, 3.0, 10000)
    assert np.allclose(O.gelu_tanh(x) - O.gelu_tanh(-x), x, rtol=1e-14, atol=1e-14)


def test_gelu_limits():
    assert O.gelu_tanh(0.0) == 0.0
    assert abs(O.gelu_tanh(20.0) - 20.0) <= 1e-12
    assert abs(O.gelu_tanh(-20.0)) <= 1e-12
    # 0.5 (1 + tanh(u)) is 1/2 at the origin: slope 1/2
    h = 1e-6
    assert abs((O.gelu_tanh(h) - O.gelu_tanh(-h)) / (2 * h) - 0.5) < 1e-9


def test_gelu_input_is_bf16_of_fp32_value():
    x = np.random.default_rng(1).normal(0.0, 2.0, 5000).astype(np.float32)
    g = O.gelu_input(x)
    assert g.dtype == np.float32
    bits = g.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "values must be bf16 values"
    # within half a bf16 step of the float64 value (plus the fp32 step)
    ref = O.gelu_tanh(x.astype(np.float64))
    step = np.where(ref != 0, 2.0 ** (np.floor(np.log2(np.abs(ref) + 1e-300)) - 7), 0)
    assert np.all(np.abs(g - ref) <= 0.5 * step * (1 + 2 ** -15) + 1e-45)
    assert np.array_equal(F.bf16_bits(F.fl32(ref)), (bits >> 16).astype(np.uint16))


def test_admissible_group_check():
    """The GPU GELU test's check for groups holding an element near a bf16
    midpoint: it accepts the quantization of either neighbour of that element
    and rejects a group whose codes match neither."""
    from tests.test_gpu_gelu import admissible, ambiguous, neighbours
    rng = np.random.default_rng(3)
    x = rng.normal(0.0, 2.0, 200000).astype(np.float32)
    amb = ambiguous(x)
    k = int(np.nonzero(amb)[0][0])
    row = rng.normal(0.0, 1.0, 64).astype(np.float32)
    row[5] = x[k]                                    # one ambiguous element in the group
    assert ambiguous(row)[5]
    xg = O.gelu_input(row)
    lo, hi = neighbours(row)
    assert lo[5] != hi[5] and xg[5] in (lo[5], hi[5])
    smooth = np.ones(64, np.float32)

    def q(v):
        c, s = O.quantize_activations(v[None, :], smooth)
        return O.pack_int4(c).tobytes() + s.view(np.uint32).tobytes()

    idx = np.nonzero(ambiguous(row))[0]
    for pick in (lo, hi):
        v = xg.copy()
        v[idx] = pick[idx]
        assert admissible(xg.copy(), lo, hi, idx, q, q(v))
    bad = bytearray(q(xg))
    bad[0] ^= 0x01                                   # a code no choice gives
    assert not admissible(xg.copy(), lo, hi, idx, q, bytes(bad))
