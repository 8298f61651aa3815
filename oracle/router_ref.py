"""Gate projection and the six-step routing epilogue, as plain float64 definitions.

TEST INFRASTRUCTURE (CPU oracle); see the package docstring.

Gate projection (commit 04cf8ca8, dsv4/layers/router.py, paragraph on the
NVFP4 gate: the gate GEMM runs on NVFP4 operands instead of bf16): logits
L[t, e] = sum_d xhat[t, d] * what[e, d], where xhat and what are the exact
dequantized NVFP4 values (code value * block scale * global scale). The
oracle takes the dequantization exactly and the dot product in float64; it
also returns A[t, e] = sum_d |xhat[t, d]| * |what[e, d]|, the scale that the
fp32-accumulation tolerance is relative to.

Epilogue (commit e0f60b9f, dsv4/kernels/router/__init__.py, paragraph on the
working path: one fused single-pass kernel doing six steps; the steps are
this router's reading, and the sorted output follows the selection sort of
commit 04cf8ca8's fused-kernel fix):

1. s = sigmoid(L) = 1 / (1 + exp(-L))
2. b = s + bias[e]                       (selection score only)
3. idx = the k experts with the largest b, in descending b, an exact tie
   going to the lower expert index
4. s_sel = s[idx]                        (the unbiased scores)
5. w = s_sel / sum(s_sel)
6. w = w * routed_scale
"""

import numpy as np

from .quant_ref import dequant_ref, quantize_ref


def logits_ref(x_codes, x_scales, gsa, w_codes, w_scales, gsw):
    """(L, A): float64 [T, E] logits and their absolute-product scale."""
    xv = dequant_ref(x_codes, x_scales, gsa)
    wv = dequant_ref(w_codes, w_scales, gsw)
    return xv @ wv.T, np.abs(xv) @ np.abs(wv).T


def sigmoid_ref(L):
    """Logistic function in float64 (overflow of exp gives the exact limit 0)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(L, dtype=np.float64)))


def route_ref(L, bias, k, routed_scale):
    """Six-step epilogue on float64 logits [T, E].

    Returns ``(idx [T,k] int64, w [T,k] float64, s [T,E], b [T,E])``.
    """
    L = np.atleast_2d(np.asarray(L, dtype=np.float64))
    T, E = L.shape
    assert 1 <= k <= E
    s = sigmoid_ref(L)
    b = s + np.asarray(bias, dtype=np.float64)[None, :]
    # Sort key (-b, index): lexsort's last key is the primary one.
    experts = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((experts, -b), axis=-1)
    idx = order[:, :k]
    s_sel = np.take_along_axis(s, idx, axis=1)
    w = float(routed_scale) * s_sel / s_sel.sum(axis=1, keepdims=True)
    return idx.astype(np.int64), w, s, b


def router_ref(x_bits, w_bits, bias, k, routed_scale, gsa_override=None):
    """Whole path from bf16 x [T, D] and bf16 gate weights [E, D].

    The gate weights are quantized by the same runtime rule (their own
    global scale gsw), as the pages do for bf16 gate and lm_head weights at
    load time (commit df05289d, dsv4/layers/grouped_linear.py, lm_head item).
    """
    xq = quantize_ref(x_bits, gsa_override)
    wq = quantize_ref(w_bits)
    L, A = logits_ref(xq[0], xq[1], xq[2], wq[0], wq[1], wq[2])
    idx, w, s, b = route_ref(L, bias, k, routed_scale)
    return {"xq": xq, "wq": wq, "L": L, "A": A, "idx": idx, "w": w, "s": s, "b": b}
