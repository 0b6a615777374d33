"""Number formats used by the method, written from their definitions (test
infrastructure only; see the package docstring).

All functions take and return NumPy arrays.  Rounding is always
round-to-nearest, ties-to-even, implemented by comparing against the exact
midpoint of the two neighbouring representable values (every midpoint used
here is exactly representable in float64, so the comparison is exact).

* fp32 ("fl32"): IEEE binary32; NumPy's float64 -> float32 cast is the IEEE
  conversion and is used as the primitive.
* bf16: the top 16 bits of a binary32 (8 exponent bits, 7 stored mantissa
  bits).  The low-rank branch is "16-bit" (aiphreaks.com page, "Technical
  Breakdown"; chaosnode.de page, "Die Technik: SVDQuant"); bf16 is the reading.
* E4M3 ("FP8 E4M3FN", OCP 8-bit float): 1 sign, 4 exponent (bias 7), 3
  mantissa bits; subnormals m * 2^-9; no infinities; 0x7F/0xFF are NaN; the
  largest finite value is 448.  Used for NVFP4 block scales.
* E2M1 (OCP FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; the eight
  magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  NVFP4 is named on the
  aiphreaks.com page ("Technical Breakdown") and the chaosnode.de page
  ("Hardware-Support").
"""

import numpy as np

F32 = np.float32
F64 = np.float64


def fl32(x):
    """Round to IEEE binary32 (round-to-nearest-even)."""
    return np.asarray(x, dtype=F64).astype(F32)


def rne_int(x):
    """Round to the nearest integer, halfway cases to the even integer."""
    return np.rint(np.asarray(x, dtype=F64))


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def bf16_bits(x):
    """binary32 values -> bf16 bit patterns (uint16), RNE; NaN stays NaN,
    overflow goes to +-inf."""
    x = fl32(x)
    u = x.view(np.uint32).astype(np.uint64)
    sign = u & 0x80000000
    mag = u & 0x7FFFFFFF
    lo = mag & 0xFFFF0000                      # truncated magnitude
    hi = lo + 0x10000                          # next bf16 magnitude up
    lo_v = (lo.astype(np.uint32)).view(F32).astype(F64)
    # spacing of bf16 values at lo: 2^(E-134) for exponent field E >= 1,
    # 2^-133 for subnormals; hi = lo + spacing (2^128 past the top, which
    # rounds to infinity as IEEE prescribes)
    e_field = ((lo >> 23) & 0xFF).astype(np.int64)
    step = np.ldexp(1.0, np.where(e_field == 0, -133, e_field - 134))
    mid = lo_v + 0.5 * step
    v = np.abs(x.astype(F64))
    lo_even = ((lo >> 16) & 1) == 0
    take_hi = (v > mid) | ((v == mid) & ~lo_even)
    res = np.where(take_hi, hi, lo)
    is_nan = np.isnan(x)
    res = np.where(is_nan, 0x7FC00000, res | sign)
    return (res >> 16).astype(np.uint16)


def bf16_to_f32(bits):
    """bf16 bit patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(F32)


def bf16(x):
    """Round binary32/float64 input to bf16, returned as float64 values.
    float64 input is first rounded to binary32 (two roundings, as the
    method states them)."""
    return bf16_to_f32(bf16_bits(fl32(x))).astype(F64)


# --------------------------------------------------------------------------
# grid rounding shared by the two small float formats
# --------------------------------------------------------------------------

def _round_to_grid(v, grid):
    """Index of the nearest grid value to each non-negative v (ties to the
    even index, saturating at the last grid point).  grid: sorted float64."""
    v = np.asarray(v, dtype=F64)
    i = np.searchsorted(grid, v, side="right") - 1          # grid[i] <= v
    i = np.clip(i, 0, len(grid) - 1)
    top = i == len(grid) - 1
    j = np.minimum(i + 1, len(grid) - 1)
    mid = 0.5 * (grid[i] + grid[j])
    up = (v > mid) | ((v == mid) & (i % 2 == 1))
    return np.where(top, len(grid) - 1, np.where(up, j, i))


# --------------------------------------------------------------------------
# E4M3 (FP8, no infinities, max 448)
# --------------------------------------------------------------------------

def _e4m3_table():
    vals = []
    for code in range(0x7F):                                 # 0x7F is NaN
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8))
    return np.array(vals, dtype=F64)


E4M3_POS = _e4m3_table()          # index == code, strictly increasing
E4M3_MAX = 448.0


def e4m3_encode(x):
    """Values -> E4M3 codes (uint8), RNE, saturating to +-448; NaN -> 0x7F.
    The sign bit is kept, so a negative value that rounds to zero gives 0x80."""
    x = np.asarray(x, dtype=F64)
    mag = np.abs(x)
    code = _round_to_grid(np.minimum(mag, E4M3_MAX), E4M3_POS).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def e4m3_decode(code):
    code = np.asarray(code, dtype=np.uint8)
    mag = code & 0x7F
    v = np.where(mag == 0x7F, np.nan, E4M3_POS[np.minimum(mag, 0x7E)])
    return np.where(code & 0x80, -v, v)


# --------------------------------------------------------------------------
# E2M1 (FP4)
# --------------------------------------------------------------------------

E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=F64)


def e2m1_encode(x):
    """Values -> 4-bit E2M1 codes (sign<<3 | magnitude index), RNE,
    saturating to +-6.  A value that rounds to zero gets code 0 (never the
    negative-zero code 0x8)."""
    x = np.asarray(x, dtype=F64)
    idx = _round_to_grid(np.abs(x), E2M1_POS).astype(np.uint8)
    neg = (x < 0) & (idx != 0)
    return np.where(neg, idx | 8, idx).astype(np.uint8)


def e2m1_decode(code):
    code = np.asarray(code, dtype=np.uint8)
    v = E2M1_POS[code & 7]
    return np.where(code & 8, -v, v)
