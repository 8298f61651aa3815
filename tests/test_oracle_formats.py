"""Pins for the E2M1 / E4M3FN tables and the nearest-rounding rule of the oracle."""

from fractions import Fraction

import numpy as np

from oracle.formats import (E2M1_GRID, E4M3_GRID, E4M3_MAX, e2m1_decode, e4m3_decode, round_to_grid,
                            round_to_grid_exact)


def test_e2m1_value_set():
    # The published E2M1 value set (OCP microscaling formats): 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    assert E2M1_GRID.tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert e2m1_decode(c | 8) == -e2m1_decode(c) or (c == 0 and e2m1_decode(8) == 0.0)
    assert np.copysign(1.0, e2m1_decode(8)) == -1.0  # code 0x8 is negative zero


def test_e4m3fn_table():
    # 127 finite non-negative values, strictly increasing with the byte.
    assert E4M3_GRID.size == 127
    assert np.all(np.diff(E4M3_GRID) > 0)
    # Largest finite value 448: the block-scale ceiling of the runtime-gsa fix
    # (commit 04cf8ca8, dsv4/layers/router.py).
    assert E4M3_MAX == 448.0 and E4M3_GRID[0x7E] == 448.0
    assert np.isnan(e4m3_decode(0x7F)) and np.isnan(e4m3_decode(0xFF))
    assert E4M3_GRID[1] == 2.0 ** -9  # smallest subnormal
    assert E4M3_GRID[8] == 2.0 ** -6  # smallest normal
    assert e4m3_decode(0x38) == 1.0 and e4m3_decode(0x58) == 16.0 and e4m3_decode(0x59) == 18.0
    # Independent closed form: every value is (8+m)/8 * 2^(e-7) for normals, m/8 * 2^-6 subnormal.
    for byte in range(127):
        e, m = byte >> 3, byte & 7
        want = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
        assert Fraction(float(E4M3_GRID[byte])) == want
        assert e4m3_decode(byte | 0x80) == -float(want) or byte == 0


def _probe_values(grid, rng):
    """Grid points, exact midpoints, their float64 neighbours, randoms and far-out values."""
    mids = (grid[:-1] + grid[1:]) / 2
    pts = np.concatenate([grid, mids])
    near = np.concatenate([np.nextafter(pts, np.inf), np.nextafter(pts, -np.inf)])
    rand = rng.uniform(0, grid[-1] * 1.2, 2000)
    logs = np.exp2(rng.uniform(np.log2(grid[1]) - 4, np.log2(grid[-1]) + 4, 2000))
    far = np.array([0.0, 1e-300, grid[-1] * 1.0000001, grid[-1] * 7, 1e30])
    return np.concatenate([pts, near[near >= 0], rand, logs, far])


def test_round_to_grid_matches_bruteforce():
    rng = np.random.default_rng(7)
    for grid in (E2M1_GRID, E4M3_GRID):
        q = _probe_values(grid, rng)
        got = round_to_grid(q, grid)
        want = [round_to_grid_exact(Fraction(float(v)), grid) for v in q]
        assert got.tolist() == want


def test_ties_go_to_even_code():
    # E2M1 midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 -> codes 0, 2, 2, 4, 4, 6, 6.
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert round_to_grid(mids, E2M1_GRID).tolist() == [0, 2, 2, 4, 4, 6, 6]
    # E4M3: 17 lies halfway between 16 (0x58) and 18 (0x59) -> 0x58; 19 -> 0x5A.
    assert round_to_grid(np.array([17.0, 19.0]), E4M3_GRID).tolist() == [0x58, 0x5A]


def test_saturation():
    assert round_to_grid(np.array([6.0, 6.5, 100.0, np.inf]), E2M1_GRID).tolist() == [7, 7, 7, 7]
    assert round_to_grid(np.array([448.0, 464.0, 480.0, 1e6]), E4M3_GRID).tolist() == [0x7E] * 4
