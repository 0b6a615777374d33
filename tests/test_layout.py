"""The device INT4 code layout (fold format) and the textbook nibble
layouts: a hand-worked chunk, the package converter against the tests' own
bit-array implementation, round trips and rejection of invalid fields.  CPU
only."""

import os

import numpy as np
import pytest

from oracle import svdq as O
from w4a4_quantized_diffusion_amd import layout
from tests.gpu_helpers import gm_int4, rm_int4

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    with open(os.path.join(HERE, "golden", "int4_fold_chunk.txt")) as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    return np.array([int(b, 16) for b in rows[0].split()], dtype=np.uint8)


def _golden_codes():
    q = np.zeros((1, 64), np.int8)
    q[0, 0], q[0, 1], q[0, 32], q[0, 37] = 1, -1, 7, -5
    return q


def test_hand_worked_chunk():
    want = _golden()
    packed = O.pack_int4(_golden_codes())
    assert np.array_equal(layout.int4_to_device(packed).reshape(-1), want)
    assert np.array_equal(gm_int4(packed).reshape(-1), want)
    assert np.array_equal(layout.int4_from_device(want.reshape(1, 1, 32)), packed)
    assert np.array_equal(rm_int4(want.reshape(1, 1, 32)), packed)


@pytest.mark.parametrize("rows,k,seed", [(1, 64, 0), (7, 192, 1), (33, 1024, 2)])
def test_two_implementations_agree_and_round_trip(rows, k, seed):
    g = np.random.default_rng(seed)
    q = g.integers(-7, 8, (rows, k)).astype(np.int8)
    q[0, :] = 7
    if rows > 1:
        q[1, :] = -7
    packed = O.pack_int4(q)
    dev = layout.int4_to_device(packed)
    assert dev.shape == (k // 64, rows, 32)
    assert np.array_equal(dev, gm_int4(packed))
    assert np.array_equal(layout.int4_from_device(dev), packed)
    assert np.array_equal(rm_int4(dev), packed)
    assert np.array_equal(O.unpack_int4(rm_int4(dev)), q)


def test_every_field_position_moves_one_code():
    """Each of the 64 codes of a group, set alone to -7, lands in exactly its
    own field (three magnitude bits and the sign) and decodes back."""
    for k in range(64):
        q = np.zeros((1, 64), np.int8)
        q[0, k] = -7
        dev = layout.int4_to_device(O.pack_int4(q))
        bits = np.unpackbits(dev.reshape(-1)).sum()
        assert bits == 4, (k, bits)
        assert np.array_equal(O.unpack_int4(layout.int4_from_device(dev)), q)


def test_negative_zero_is_rejected():
    """A field with the sign set and magnitude 0 is the one bit pattern that
    is no code: the tests' decoder keeps it visible (nibble 0x8), the package
    converter raises, in both directions."""
    neg0 = np.zeros((1, 1, 32), np.uint8)
    neg0[0, 0, 0] = 0x20                # bit 5 of X: the sign of field 0, magnitude 0
    assert rm_int4(neg0)[0, 0] == 0x08
    with pytest.raises(ValueError):
        layout.int4_from_device(neg0)
    with pytest.raises(ValueError):
        layout.int4_to_device(np.array([[0x08] + [0] * 31], np.uint8))


def test_textbook_group_major_round_trip():
    g = np.random.default_rng(3)
    packed = g.integers(0, 256, (5, 96), dtype=np.uint8)
    dev = layout.nibbles_to_device(packed)
    assert dev.shape == (3, 5, 32)
    assert np.array_equal(layout.nibbles_from_device(dev), packed)
