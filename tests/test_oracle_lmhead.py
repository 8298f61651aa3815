"""Pins of the greedy lm_head oracle: a one-hot hand case with an exact tie,
brute force over rows with exact rational dot products, and planted mistakes
that its checker must catch."""

from fractions import Fraction

import numpy as np

from nvfp4_block_scaled_06_amd import workloads as wl
from oracle import lmhead_ref, quant_ref


def q(a):
    """Quantize fp64 values after rounding them to bf16 (the hand case's values are bf16-exact)."""
    return quant_ref.quantize_ref(wl.bf16_bits(np.asarray(a, dtype=np.float32)))


def test_one_hot_tie_goes_to_lower_row():
    # x = [2688, 0...]: gsa = 1, scale 448, code 6. Rows 3 and 5 hold 2688 at element 0 (gsw = 1), so both
    # logits are 2688 * 2688 = 7,225,344 exactly; row 1 holds 1344 (half), row 2 is negative.
    D, N = 32, 6
    x = np.zeros((1, D)); x[0, 0] = 2688.0
    w = np.zeros((N, D)); w[1, 0] = 1344.0; w[2, 0] = -2688.0; w[3, 0] = 2688.0; w[5, 0] = 2688.0
    idx, top, L, A = lmhead_ref.lmhead_ref(*q(x), *q(w))
    assert idx.tolist() == [3]
    assert top.tolist() == [7225344.0]
    assert L[0].tolist() == [0.0, 3612672.0, -7225344.0, 7225344.0, 0.0, 7225344.0]


def test_brute_force_exact_rationals():
    rng = np.random.default_rng(7)
    T, D, N = 3, 64, 40
    x = rng.standard_normal((T, D))
    w = 0.02 * rng.standard_normal((N, D))
    xq, wq = q(x), q(w)
    idx, top, L, A = lmhead_ref.lmhead_ref(*xq, *wq)
    xv = quant_ref.dequant_ref(*xq)
    wv = quant_ref.dequant_ref(*wq)
    for t in range(T):
        exact = [sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[t], wv[n])) for n in range(N)]
        best = max(range(N), key=lambda n: (exact[n], -n))
        assert idx[t] == best
        # float64 summation: within D ulps of the condition scale of the exact value.
        assert abs(float(Fraction(float(top[t])) - exact[best])) <= D * 2.0 ** -52 * A[t, best]


def test_checker_catches_planted_mistakes():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((4, 50)) * 10
    A = np.abs(L) + 1.0
    idx, top = lmhead_ref.argmax_ref(L)
    assert lmhead_ref.check_argmax(idx, top, L, A) == []
    wrong = idx.copy(); wrong[2] = (wrong[2] + 1) % 50
    assert lmhead_ref.check_argmax(wrong, L[np.arange(4), wrong], L, A)  # a clearly smaller row
    off = top.copy(); off[1] += 1e-3 * A[1, idx[1]]
    assert lmhead_ref.check_argmax(idx, off, L, A)  # logit outside tolerance
    # Near-tie: a second row within tolerance of the maximum may be chosen instead.
    L2 = L.copy(); j = (idx[0] + 7) % 50; L2[0, j] = top[0] - 1e-7 * A[0, j]
    assert lmhead_ref.check_argmax(np.array([j, *idx[1:]]), np.array([L2[0, j], *top[1:]]), L2, A) == []
