"""AWQ-style W4A16 linear layer (weight-only INT4): the oracle (test
infrastructure only; see the package docstring).

The chaosnode.de page ("Nunchaku Lite vs. Original", "Hardware-Support")
names awq_w4a16 / INT4 as the second layer type that Nunchaku Lite patches
into a model next to svdq_w4a4; it gives no recipe.  The reading used here is
plain asymmetric round-to-nearest INT4 with groups of 64 along K, bf16 scales
and bf16 zero points (the activation-aware scale search needs calibration
data and is not part of this layer).

For each output row n and group of 64 weights w:
  mn = min(min w, 0),  mx = max(max w, 0)
  s  = bf16(fl32(fl32(mx - mn) / 15))
  s == 0: z = 0, q = 0
  else:   z = clamp(rne(fl32(-mn / s)), 0, 15)
          q = clamp(rne(fl32(w / s)) + z, 0, 15)
Codes are unsigned nibbles, two per byte, even k in the low nibble.  A zero
point is an integer; zero is stored as +0.

W4A16 means 4-bit storage and a 16-bit multiply.  The pages leave the
precision of the dequantized weight open; the reading used here is the
activations' type: wd = bf16((q - z) s), rounded once from the exact product
(4-bit integer times 8-bit significand).  Then
Y = X @ wd^T + b, summed exactly (float64).
"""

import numpy as np

from .formats import fl32, bf16, bf16_bits, rne_int
from .svdq import pack_nibbles, unpack_nibbles

F64 = np.float64
GROUP = 64


def quantize_weights(w, group=GROUP):
    """Returns (q uint8 [N, K] values 0..15, s float64 bf16 values [N, K/g],
    z float64 integer values [N, K/g], packed codes [N, K/2])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % group == 0
    wg = w.reshape(n, k // group, group).astype(F64)
    mn = np.minimum(np.min(wg, axis=2), 0.0)
    mx = np.maximum(np.max(wg, axis=2), 0.0)
    s = bf16(fl32(fl32(mx - mn).astype(F64) / 15.0))
    sd = s[:, :, None]
    safe = np.where(sd > 0, sd, 1.0)
    z = np.where(s > 0, np.clip(rne_int(fl32(-mn / np.where(s > 0, s, 1.0))), 0, 15), 0.0)
    z = z + 0.0                              # an integer: -0 becomes +0
    q = np.where(sd > 0,
                 np.clip(rne_int(fl32(wg / safe)) + z[:, :, None], 0, 15), 0.0)
    q = q.reshape(n, k).astype(np.uint8)
    return q, s, z, pack_nibbles(q)


def dequantize(q, s, z, group=GROUP):
    n, k = q.shape
    qg = np.asarray(q, dtype=F64).reshape(n, k // group, group)
    return ((qg - z[:, :, None]) * s[:, :, None]).reshape(n, k)


def dequantize_bf16(q, s, z, group=GROUP):
    """The 16-bit weights the multiply uses: bf16((q - z) s)."""
    return bf16(dequantize(q, s, z, group))


def linear_w4a16(x, q, s, z, bias=None, group=GROUP):
    """Y = X @ bf16((q - z) s)^T + b in float64.  x: [M, K] float32 values
    (bf16 inputs passed as their values)."""
    wd = dequantize_bf16(q, s, z, group)
    y = np.asarray(x, dtype=F64) @ wd.T
    if bias is not None:
        y += np.asarray(bias, dtype=F64)[None, :]
    return y


def scales_bits(s):
    return bf16_bits(fl32(s))


def unpack(packed):
    return unpack_nibbles(packed)
