"""Pins of the oracle's number formats against independent references:
torch's CPU conversions (bf16, float8_e4m3fn), hand-worked tie tables from
the format definitions, and exhaustive brute force over small grids."""

import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append([float(t) for t in line.split()])
    return np.array(rows)


def test_bf16_matches_torch_on_random_bit_patterns():
    g = np.random.default_rng(1)
    u = g.integers(0, 2 ** 32, size=500_000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000,
                         0x00018000, 0x3F808000, 0x3F818000, 0x7F800000, 0xFF800000,
                         0x00000001, 0x807FFFFF], dtype=np.uint32)
    x = np.concatenate([u, specials]).view(np.float32)
    x = x[~np.isnan(x)]
    ours = F.bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even is 1.0
    assert F.bf16(np.float32(1 + 2 ** -8)) == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: even is 1 + 2^-6
    assert F.bf16(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6


def test_e4m3_table_closed_form():
    t = F.E4M3_POS
    assert len(t) == 127 and t[0] == 0 and t[-1] == 448.0
    assert t[1] == 2.0 ** -9 and t[8] == 2.0 ** -6      # smallest subnormal / normal
    assert np.all(np.diff(t) > 0)


def test_e4m3_matches_torch_including_all_midpoints():
    g = np.random.default_rng(2)
    v = (g.standard_normal(200_000) * 60).astype(np.float32)
    grid = F.E4M3_POS
    mids = 0.5 * (grid[1:] + grid[:-1])
    v = np.concatenate([v, grid, mids, -mids, grid * 1.0000001]).astype(np.float32)
    ours = F.e4m3_encode(v)
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    back = F.e4m3_decode(ours)
    assert np.all(np.abs(back) <= 448)


def test_e4m3_saturates():
    assert F.e4m3_encode(np.array([1e6, 480.0, 464.0]))[0] == 0x7E
    assert np.all(F.e4m3_decode(F.e4m3_encode(np.array([1e6, 480.0, 464.0]))) == 448.0)


def test_e2m1_tie_table():
    rows = _load("e2m1_ties.txt")
    codes = F.e2m1_encode(rows[:, 0])
    assert np.array_equal(codes, rows[:, 2].astype(np.uint8))
    assert np.array_equal(F.e2m1_decode(codes), rows[:, 1])


def test_e2m1_brute_force_nearest():
    # exhaustive: for many values the chosen grid point is at minimal distance
    g = np.random.default_rng(3)
    v = g.uniform(-7, 7, 100_000)
    dec = F.e2m1_decode(F.e2m1_encode(v))
    cand = np.concatenate([F.E2M1_POS, -F.E2M1_POS])
    best = np.min(np.abs(v[:, None] - cand[None, :]), axis=1)
    assert np.all(np.abs(v - dec) <= best + 0.0)
    assert np.all(F.e2m1_encode(v[np.abs(v) < 0.25]) == 0)


def test_rne_int_halves():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.4999999, 6.5, -6.5])
    assert list(F.rne_int(x)) == [0, 2, 2, 0, -2, -2, 3, 6, -6]


@pytest.mark.parametrize("x", [1.0 / 3.0, 2.0 / 7.0, 1e-40, 3.4e38])
def test_fl32_is_ieee_cast(x):
    assert F.fl32(x) == np.float32(x)
