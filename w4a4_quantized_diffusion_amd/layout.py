"""Host-side converters between the textbook 4-bit packing and the
library's device code layouts (argument marshalling, NumPy only).

The library's own quantizers (svdq_quantize_weights, svdq_act_quantize)
write the device layouts directly; these helpers are for callers that bring
codes from elsewhere, and for inspecting what the library wrote.

Textbook packing: [rows, K/2] bytes, two codes per byte, even k in the low
nibble; an INT4 code q in -7..7 is the sign-magnitude nibble
|q| | (q < 0) << 3 (zero is 0x0).

Device layouts are group-major along K: the 32 bytes of (group g, row r)
sit at byte offset (g * rows + r) * 32.

  * NVFP4 (E2M1 nibbles) and AWQ (unsigned nibbles): the row's 64 codes of
    the group in textbook order.
  * INT4 ("fold" format): the 32 bytes are four 8-byte chunks.  Chunk c
    holds the codes k = 8c + j as fields j and k = 32 + 8c + j as fields
    8 + j (j = 0..7).  Field f is the 6-bit pattern |q| | (q < 0) << 5 (the
    code as an FP6-E2M3 subnormal, q / 8) at bits 6f .. 6f + 5 of a 96-bit
    string with words o0, o1, o2.  The chunk stores the little-endian words
    X = o0 | (o1 & GX) and Y = o2 | (o1 & GY), GX = 0x18618618 and
    GY = 0x61861861: GX marks the exponent bits of o0's fields, GY those of
    o2's, and together they are exactly o1's payload bits, so
    o0 = X & ~GX, o2 = Y & ~GY, o1 = (X & GX) | (Y & GY).
"""

import numpy as np

GX = 0x18618618
GY = 0x61861861
_M32 = np.uint64(0xFFFFFFFF)


def _nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    nib = np.empty((rows, 2 * half), dtype=np.uint8)
    nib[:, 0::2] = packed & 15
    nib[:, 1::2] = packed >> 4
    return nib


def _pack(nib):
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def nibbles_to_device(packed):
    """Textbook packing [rows, K/2] -> group-major [K/64, rows, 32] (the
    NVFP4 and AWQ device layout)."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    if half % 32:
        raise ValueError("K must be a multiple of 64")
    return np.ascontiguousarray(packed.reshape(rows, half // 32, 32).transpose(1, 0, 2))


def nibbles_from_device(dev):
    """Group-major [K/64, rows, 32] -> textbook packing [rows, K/2]."""
    dev = np.asarray(dev, dtype=np.uint8)
    g, rows, width = dev.shape
    if width != 32:
        raise ValueError("expected [K/64, rows, 32] bytes")
    return np.ascontiguousarray(dev.transpose(1, 0, 2).reshape(rows, g * 32))


def int4_to_device(packed):
    """INT4 codes in the textbook packing [rows, K/2] (sign-magnitude
    nibbles) -> the fold format, group-major [K/64, rows, 32] bytes."""
    nib = _nibbles(packed)
    rows, k = nib.shape
    if k % 64:
        raise ValueError("K must be a multiple of 64")
    g = k // 64
    if np.any(nib == 8):
        raise ValueError("negative zero nibble 0x8 is not a valid INT4 code")
    f = ((nib & 7) | ((nib >> 3) << 5)).astype(np.uint64)
    # [rows, g, half, c, j] with k = 32 half + 8 c + j -> [g, rows, c, field]
    f = f.reshape(rows, g, 2, 4, 8).transpose(1, 0, 3, 2, 4).reshape(g, rows, 4, 16)
    lo = np.zeros(f.shape[:-1], dtype=np.uint64)     # string bits 0..63
    hi = np.zeros(f.shape[:-1], dtype=np.uint64)     # string bits 64..95
    for fi in range(16):
        b = 6 * fi
        if b + 6 <= 64:
            lo |= f[..., fi] << np.uint64(b)
        elif b >= 64:
            hi |= f[..., fi] << np.uint64(b - 64)
        else:                                        # field 10 straddles bit 64
            lo |= (f[..., fi] << np.uint64(b)) & np.uint64(0xFFFFFFFFFFFFFFFF)
            hi |= f[..., fi] >> np.uint64(64 - b)
    o0, o1, o2 = lo & _M32, lo >> np.uint64(32), hi
    x = (o0 | (o1 & np.uint64(GX))).astype(np.uint32)
    y = (o2 | (o1 & np.uint64(GY))).astype(np.uint32)
    words = np.stack([x, y], axis=-1)                # [g, rows, 4, 2]
    return np.ascontiguousarray(words.astype("<u4").view(np.uint8).reshape(g, rows, 32))


def int4_from_device(dev):
    """Fold-format INT4 codes [K/64, rows, 32] -> textbook packing
    [rows, K/2].  Every 64-bit chunk decodes to sixteen fields with zero
    exponent bits; a field with the sign set and magnitude 0 (negative zero,
    which no quantizer writes) raises."""
    dev = np.ascontiguousarray(np.asarray(dev, dtype=np.uint8))
    g, rows, width = dev.shape
    if width != 32:
        raise ValueError("expected [K/64, rows, 32] bytes")
    w = dev.view("<u4").reshape(g, rows, 4, 2).astype(np.uint64)
    x, y = w[..., 0], w[..., 1]
    o0 = x & np.uint64(~GX & 0xFFFFFFFF)
    o2 = y & np.uint64(~GY & 0xFFFFFFFF)
    o1 = (x & np.uint64(GX)) | (y & np.uint64(GY))
    lo = o0 | (o1 << np.uint64(32))
    fields = []
    for fi in range(16):
        b = 6 * fi
        if b + 6 <= 64:
            v = lo >> np.uint64(b)
        elif b >= 64:
            v = o2 >> np.uint64(b - 64)
        else:
            v = (lo >> np.uint64(b)) | (o2 << np.uint64(64 - b))
        fields.append(v & np.uint64(63))
    f = np.stack(fields, axis=-1).astype(np.uint8)   # [g, rows, c, field]
    if np.any(f == 0x20):
        raise ValueError("negative zero field: not an INT4 code")
    nib = (f & 7) | ((f >> 5) << 3)
    # [g, rows, c, half, j] -> [rows, g, half, c, j]
    nib = nib.reshape(g, rows, 4, 2, 8).transpose(1, 0, 3, 2, 4).reshape(rows, g * 64)
    return _pack(nib)
