"""Greedy lm_head reference: logits over a vocabulary-sized NVFP4 weight
matrix and the row with the largest logit.

TEST INFRASTRUCTURE (CPU oracle); see the package docstring.

The NVFP4 lm_head replaces a 1.8 GB BF16 weight (commit df05289d,
dsv4/layers/grouped_linear.py, weights paragraph). Its logits have the same
plain definition as the gate's (router_ref.logits_ref: exact float64 dot
products of the dequantized operands); greedy decoding takes the largest,
an exact tie going to the lower row (the first maximum).
"""

import numpy as np

from .router_ref import logits_ref


def argmax_ref(L):
    """Row of the largest logit per token, ties to the lower row: (idx [T] int64, logit [T])."""
    L = np.atleast_2d(np.asarray(L, dtype=np.float64))
    idx = np.argmax(L, axis=1)
    return idx.astype(np.int64), L[np.arange(L.shape[0]), idx]


def lmhead_ref(x_codes, x_scales, gsa, w_codes, w_scales, gsw):
    """(idx [T], logit [T], L [T, N], A [T, N]) for quantized x and weights."""
    L, A = logits_ref(x_codes, x_scales, gsa, w_codes, w_scales, gsw)
    idx, top = argmax_ref(L)
    return idx, top, L, A


def check_argmax(dev_idx, dev_logit, L_ref, A_ref, tol=1e-5):
    """Failures (empty == pass) of a device greedy choice against the reference logits.

    The device logit of its chosen row must match the reference within tol * A (the dot product's condition
    scale, as for the gate logits). The chosen row must be the reference's first maximum unless another row's
    logit is within tol * (A_chosen + A_best) of the maximum (a near-tie, where rounding may pick either)."""
    out = []
    L_ref = np.atleast_2d(L_ref)
    A_ref = np.atleast_2d(A_ref)
    ridx, rtop = argmax_ref(L_ref)
    for t in range(L_ref.shape[0]):
        j, r = int(dev_idx[t]), int(ridx[t])
        if not 0 <= j < L_ref.shape[1]:
            out.append(f"token {t}: row {j} out of range")
            continue
        if abs(float(dev_logit[t]) - L_ref[t, j]) > tol * A_ref[t, j]:
            out.append(f"token {t}: logit {float(dev_logit[t])!r} of row {j}, reference {L_ref[t, j]!r}")
        if j != r and L_ref[t, j] < rtop[t] - tol * (A_ref[t, j] + A_ref[t, r]):
            out.append(f"token {t}: row {j} (logit {L_ref[t, j]!r}) chosen, reference row {r} ({rtop[t]!r})")
    return out
