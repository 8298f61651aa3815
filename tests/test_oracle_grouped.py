"""Pins for the oracle's grouped NVFP4 product (group offsets, one shared activation scale, per-group weights)."""

from fractions import Fraction

import numpy as np

from conftest import bf16_exact, hex_bytes, load_golden
from nvfp4_block_scaled_06_amd import workloads as wl
from oracle import check
from oracle.formats import E2M1_GRID, E4M3_GRID
from oracle.grouped_ref import grouped_products, grouped_ref, offsets_ref
from oracle.quant_ref import quantize_ref, unpack_codes

GOLD = load_golden("grouped_worked_examples.json")


def test_offsets_closed_form():
    c = GOLD["offsets"]
    assert offsets_ref(c["G"], c["padded_rows"]).tolist() == c["expect"]
    assert offsets_ref(5, 0).tolist() == [0] * 6


def _case(name):
    c = GOLD[name]
    x = np.stack([bf16_exact(r) for r in c["x"]])
    w = np.stack([np.stack([bf16_exact(r) for r in wg]) for wg in c["w"]])
    return c, x, w


def test_per_group_weight_scales():
    c, x, w = _case("per_group_weight_scale")
    r = grouped_ref(x, c["offsets"], w)
    assert [float(q[2]) for q in r["wq"]] == c["expect_gsw"]
    assert r["Y"].tolist() == c["expect_Y"]
    assert r["A"].tolist() == c["expect_A"]


def test_one_activation_scale_for_all_groups():
    """An outlier in group 1 sets the scale group 0 is quantized with."""
    c, x, w = _case("shared_activation_scale")
    r = grouped_ref(x, c["offsets"], w)
    assert float(r["xq"][2]) == c["expect_gsa"]
    assert r["xq"][1][:, 0].tolist() == [int(h, 16) for h in c["expect_scales_hex"]]
    assert r["Y"].tolist() == c["expect_Y"]
    # Group 0 on its own would have been quantized with gsa 1 and scale 0x7E.
    alone = quantize_ref(x[:1])
    assert float(alone[2]) == 1.0 and int(alone[1][0, 0]) == 0x7E


def _exact_grouped(xq, wq, offsets):
    """Y as exact Fractions from the integer codes: gsa gsw_g sum_b S_x S_w sum_i (2 q_x)(2 q_w) / 4."""
    xc, xs, gsa = xq
    ux = unpack_codes(xc).astype(int)

    def twice(code):
        m = int(round(2 * E2M1_GRID[code & 7]))
        return -m if code & 8 else m

    R, D = ux.shape
    out = {}
    for g in range(len(offsets) - 1):
        wc, ws, gsw = wq[g]
        uw = unpack_codes(wc).astype(int)
        for r in range(offsets[g], offsets[g + 1]):
            for n in range(uw.shape[0]):
                acc = Fraction(0)
                for b in range(D // 16):
                    isum = sum(twice(ux[r, 16 * b + i]) * twice(uw[n, 16 * b + i]) for i in range(16))
                    acc += Fraction(isum, 4) * Fraction(float(E4M3_GRID[xs[r, b]])) * Fraction(float(E4M3_GRID[ws[n, b]]))
                out[(r, n)] = acc * Fraction(float(gsa)) * Fraction(float(gsw))
    return out


def test_brute_force_tiny_groups_with_an_empty_group():
    rng = np.random.default_rng(31)
    offsets = [0, 2, 2, 5]  # group 1 has no rows
    x = wl.bf16_bits(rng.standard_normal((6, 32)).astype(np.float32))  # row 5 belongs to no group
    w = wl.bf16_bits((rng.standard_normal((3, 4, 32)) * np.array([1.0, 0.01, 30.0])[:, None, None]).astype(np.float32))
    r = grouped_ref(x, offsets, w)
    exact = _exact_grouped(r["xq"], r["wq"], offsets)
    assert len(exact) == 5 * 4
    for (row, n), v in exact.items():
        assert abs(Fraction(float(r["Y"][row, n])) - v) <= Fraction(float(r["A"][row, n])) * Fraction(1, 2 ** 40)
    assert np.all(np.isnan(r["Y"][5]))  # no group: no defined output
    # Different weight scales per group (the groups' magnitudes differ by 100 and 3000).
    gsw = [float(q[2]) for q in r["wq"]]
    assert gsw[1] < gsw[0] < gsw[2]


def test_row_subset_matches_full_product():
    """Rows quantized under the whole tensor's scale, then multiplied one subset at a time (how the GPU tests
    check the large shapes), give the full product's rows."""
    rng = np.random.default_rng(5)
    offsets = offsets_ref(3, 7)
    x = wl.bf16_bits(rng.standard_normal((21, 64)).astype(np.float32))
    w = wl.bf16_bits((rng.standard_normal((3, 9, 64)) * 0.02).astype(np.float32))
    full = grouped_ref(x, offsets, w)
    rows = np.array([0, 6, 7, 13, 20])
    sub = quantize_ref(x[rows], gsa_override=full["xq"][2])
    part = grouped_products(sub, full["wq"], offsets, rows=rows)
    assert np.array_equal(part["Y"], full["Y"][rows]) and np.array_equal(part["A"], full["A"][rows])


def test_checker_catches_a_wrong_group_weight():
    """A product taken with the neighbouring group's weights must fail the logit-style check."""
    rng = np.random.default_rng(8)
    offsets = [0, 4, 8]
    x = wl.bf16_bits(rng.standard_normal((8, 64)).astype(np.float32))
    w = wl.bf16_bits((rng.standard_normal((2, 5, 64)) * 0.02).astype(np.float32))
    r = grouped_ref(x, offsets, w)
    swapped = grouped_products(r["xq"], r["wq"][::-1], offsets)
    assert check.check_logits(swapped["Y"], r["Y"], r["A"])
    assert not check.check_logits(r["Y"].astype(np.float32), r["Y"], r["A"])
