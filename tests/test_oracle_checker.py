"""Mutation tests: mistakes planted in oracle outputs (on the CPU) must be caught by the checker."""

import numpy as np

from nvfp4_block_scaled_06_amd import workloads as wl
from oracle.check import check_logits, check_quant, check_topk
from oracle.quant_ref import quantize_ref
from oracle.router_ref import route_ref, router_ref


def _ref(cfg=1):
    c = wl.CONFIGS[cfg]
    return c, router_ref(wl.make_x(cfg), wl.make_w(cfg), wl.make_bias(cfg), c.k, c.routed_scale)


def test_quant_checker_catches_single_bit_flips():
    codes, scales, gsa = quantize_ref(wl.make_x(1))
    assert check_quant(codes, scales, gsa, (codes, scales, gsa)) == []
    c2 = codes.copy()
    c2[2, 17] ^= 0x10
    assert check_quant(c2, scales, gsa, (codes, scales, gsa))
    s2 = scales.copy()
    s2[1, 3] ^= 0x01
    assert check_quant(codes, s2, gsa, (codes, scales, gsa))
    g2 = np.nextafter(gsa, np.float32(np.inf))
    assert check_quant(codes, scales, g2, (codes, scales, gsa))


def test_logit_checker_tolerance_is_relative_to_abs_product_scale():
    c, r = _ref()
    L, A = r["L"], r["A"]
    assert check_logits(L, L, A) == []
    ok = L + 0.5e-5 * A
    assert check_logits(ok, L, A) == []
    bad = L.copy()
    bad[1, 5] += 2e-5 * A[1, 5]
    assert check_logits(bad, L, A)


def test_topk_checker_catches_wrong_set_order_and_weights():
    c, r = _ref(3)
    idx, w, s, b = r["idx"], r["w"], r["s"], r["b"]
    assert check_topk(idx, w, s, b, c.k, c.routed_scale) == []
    # Replace a chosen expert with a clearly worse one.
    t = 0
    order = np.lexsort((np.arange(c.E), -b[t]))
    bad = idx.copy()
    bad[t, -1] = order[-1]
    assert check_topk(bad, w, s, b, c.k, c.routed_scale)
    # Swap the first and last chosen experts (descending order broken by a clear margin).
    if b[t, idx[t, 0]] - b[t, idx[t, -1]] >= 1e-5:
        sw = idx.copy()
        sw[t, [0, -1]] = sw[t, [-1, 0]]
        assert check_topk(sw, w, s, b, c.k, c.routed_scale)
    # Perturb one weight by 2e-5.
    w2 = w.copy()
    w2[t, 3] += 2e-5
    assert check_topk(idx, w2, s, b, c.k, c.routed_scale)
    # Duplicate index.
    dup = idx.copy()
    dup[t, 1] = dup[t, 0]
    assert check_topk(dup, w, s, b, c.k, c.routed_scale)


def test_topk_checker_allows_either_side_of_a_near_tie():
    # Experts 1 and 2 differ by 1e-7 in b at the k/k+1 boundary: either may be chosen.
    L = np.array([[3.0, 0.0, 0.0, -3.0]])
    bias = np.array([0.0, 1e-7, 0.0, 0.0])
    idx, w, s, b = route_ref(L, bias, 2, 1.0)
    assert idx[0].tolist() == [0, 1]
    alt = np.array([[0, 2]])
    s_alt = s[0, [0, 2]]
    w_alt = (s_alt / s_alt.sum())[None, :]
    assert check_topk(alt, w_alt, s, b, 2, 1.0) == []
    # But never the clearly worse expert 3.
    bad = np.array([[0, 3]])
    s_bad = s[0, [0, 3]]
    assert check_topk(bad, (s_bad / s_bad.sum())[None, :], s, b, 2, 1.0)
    # And a weight computed on the wrong set is caught even if the set is allowed.
    assert check_topk(alt, w[:, :], s, b, 2, 1.0) or np.allclose(w, w_alt, atol=1e-5)
