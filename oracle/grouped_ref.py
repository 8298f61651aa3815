"""Grouped NVFP4 GEMM over padded groups, written as its plain definition.

TEST INFRASTRUCTURE (CPU oracle); see the package docstring.

Source: commit df05289d, ``dsv4/layers/grouped_linear.py`` (the grouped
linear layer that the router's experts and the attention output projection
use), read step by step:

1. Group offsets. Group g's rows start at g * padded_rows: the fix replaces a
   host loop that wrote each offset (one host-device sync per group) by an
   element-wise product of a range tensor [0, 1, ..., G], allocated once at
   initialization, with padded_rows (``offsets_ref``). Group g owns rows
   [offsets[g], offsets[g + 1]) of the flattened activations.
2. One quantization for all groups. The activations of every group are
   flattened into one (G * padded_rows, D) tensor and quantized in a single
   launch with one device-side global scale (``quantize_ref`` over the whole
   tensor: gsa = max|x| / 2688 over all groups, so an outlier in one group
   sets the scale of every group).
3. Each group's weight is its own NVFP4 tensor (N rows of D elements, the
   checkpoint's row-major (N, K_packed) layout) with its own global scale
   gsw[g] (here the weights are bf16 quantized at load time by the runtime
   rule, max|W_g| / 2688 per group).
4. Y[r, n] = sum_d xhat[r, d] * what_g[n, d] for every row r of group g:
   the dequantized values are exact in float64, and so is the dot product up
   to the float64 summation (error <= D * 2^-53 * A, A the sum of absolute
   products, which is also returned as the tolerance scale).

Rows at or past offsets[G] belong to no group and have no defined output
(NaN here).
"""

import numpy as np

from .quant_ref import dequant_ref, quantize_ref


def offsets_ref(G, padded_rows):
    """Group offsets [G + 1]: range(G + 1) * padded_rows (int64)."""
    return np.arange(G + 1, dtype=np.int64) * int(padded_rows)


def grouped_ref(x_bits, offsets, w_bits, gsa_override=None):
    """Whole grouped layer from bf16 x [R, D] and bf16 weights [G, N, D].

    Returns ``{"xq", "wq" (one tuple per group), "Y" [R, N] float64, "A" [R, N]}``.
    """
    x_bits = np.asarray(x_bits)
    offsets = np.asarray(offsets, dtype=np.int64)
    G = len(offsets) - 1
    R = x_bits.shape[0]
    assert offsets[0] == 0 and np.all(np.diff(offsets) >= 0) and offsets[G] <= R
    xq = quantize_ref(x_bits, gsa_override)
    wq = [quantize_ref(w_bits[g]) for g in range(G)]
    return {"xq": xq, "wq": wq, **grouped_products(xq, wq, offsets)}


def grouped_products(xq, wq, offsets, rows=None):
    """Y and A of the grouped product from quantized x and weights.

    ``xq`` holds every row, or only the rows listed in ``rows`` (global row indexes, quantized under the whole
    tensor's global scale); the result has one row per row of ``xq``."""
    offsets = np.asarray(offsets, dtype=np.int64)
    G = len(offsets) - 1
    xv = dequant_ref(*xq)
    N = wq[0][0].shape[0]
    rows = np.arange(xv.shape[0]) if rows is None else np.asarray(rows)
    assert len(rows) == xv.shape[0]
    Y = np.full((len(rows), N), np.nan)
    A = np.full((len(rows), N), np.nan)
    for g in range(G):
        sel = np.nonzero((rows >= offsets[g]) & (rows < offsets[g + 1]))[0]
        if sel.size == 0:
            continue
        wv = dequant_ref(*wq[g])
        xr = xv[sel]
        Y[sel] = xr @ wv.T
        A[sel] = np.abs(xr) @ np.abs(wv).T
    return {"Y": Y, "A": A}
