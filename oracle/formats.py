"""E2M1 and E4M3FN: decoding from bit fields and nearest rounding.

TEST INFRASTRUCTURE (CPU oracle); see the package docstring.

E2M1 (the NVFP4 element format): 1 sign bit, 2 exponent bits with bias 1,
1 mantissa bit, no infinities or NaN. Exponent field 0 is subnormal.

E4M3FN (the NVFP4 block-scale format, OCP "FN" variant): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, no infinities; only the
all-ones pattern (0x7F / 0xFF) is NaN. Its largest finite value is 448, the
block-scale ceiling the runtime-gsa fix is built around (commit 04cf8ca8,
dsv4/layers/router.py, paragraph on the checkpoint input_scale bug).

Rounding rule used for both formats (a reading the pages leave open; it is
the IEEE conversion rule): the result is the representable value nearest to
the exact real argument; an exact tie goes to the even code (even mantissa
bit); anything above the largest finite value saturates to it, which is
what "systematic magnitude loss" past 448 means on the page above.
"""

from fractions import Fraction

import numpy as np


def e2m1_decode(code):
    """Value of a 4-bit E2M1 code, from its bit fields (exact float)."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    exp_field = (code >> 1) & 0x3
    man = code & 0x1
    if exp_field == 0:
        mag = man * 0.5  # subnormal: m * 2^(1-bias) * 2^-1
    else:
        mag = (1.0 + man / 2.0) * 2.0 ** (exp_field - 1)
    return sign * mag


def e4m3_decode(byte):
    """Value of an E4M3FN byte, from its bit fields (exact float; NaN for 0x7F/0xFF)."""
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    exp_field = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp_field == 0xF and man == 0x7:
        return float("nan")
    if exp_field == 0:
        mag = man * 2.0 ** -9  # subnormal: m/8 * 2^(1-7)
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp_field - 7)
    return sign * mag


# Non-negative grids, indexed by code (code order == value order for both).
E2M1_GRID = np.array([e2m1_decode(c) for c in range(8)], dtype=np.float64)
E4M3_GRID = np.array([e4m3_decode(b) for b in range(0x7F)], dtype=np.float64)  # 0x00..0x7E
E4M3_MAX = float(E4M3_GRID[-1])
E2M1_MAX = float(E2M1_GRID[-1])


def round_to_grid(q, grid):
    """Code of the grid value nearest to each q >= 0 (float64 array).

    Ties go to the even code; values above the top of the grid saturate.
    ``grid`` is strictly increasing and the code of ``grid[i]`` is ``i``.

    The comparison is against the exact midpoints between neighbouring grid
    values (each representable in float64). It decides the rounding of the
    exact real quotient whenever ``q`` is the correctly rounded float64
    quotient of the quantizer's operands: those quotients can only sit on a
    midpoint when they equal it exactly, and otherwise stay at least ~2^-31
    (relative) away from it, far more than float64's 2^-53 rounding error.
    """
    q = np.asarray(q, dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) * 0.5
    below = np.searchsorted(mids, q, side="left")  # number of midpoints < q
    hit = below < mids.size
    tie = np.zeros(q.shape, dtype=bool)
    tie[hit] = mids[below[hit]] == q[hit]
    # A tie at midpoint j lies between codes j and j+1: keep the even one.
    up = tie & ((below + 1) % 2 == 0)
    return (below + up).astype(np.int64)


def round_to_grid_exact(q, grid):
    """Brute-force twin of ``round_to_grid`` for one exact rational q >= 0.

    Scans every grid value with exact ``Fraction`` distances; used by the
    tests on small inputs and exhaustive sweeps.
    """
    q = Fraction(q)
    best_code, best_dist = None, None
    for code, g in enumerate(grid):
        dist = abs(q - Fraction(float(g)))
        if best_dist is None or dist < best_dist or (dist == best_dist and code % 2 == 0):
            best_code, best_dist = code, dist
    return best_code
