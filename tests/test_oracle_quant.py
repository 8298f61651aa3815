"""Pins for the oracle's NVFP4 quantizer: closed forms, worked examples, sweeps, invariants."""

from fractions import Fraction

import numpy as np
import pytest

from conftest import bf16_exact, hex_bytes, load_golden
from nvfp4_block_scaled_06_amd import workloads as wl
from oracle.formats import E2M1_GRID, E4M3_GRID, round_to_grid_exact
from oracle.quant_ref import (block_scale_bytes, dequant_ref, element_codes, gsa_ref, pack_codes,
                              quantize_exact_scalar, quantize_ref, unpack_codes)


def f32_hex(v):
    return f"{int(np.array(v, dtype=np.float32).view(np.uint32)):08X}"


def f32_nearest_exact(q):
    """Exact nearest-even fp32 to a positive rational, by comparing the two fp32 neighbours."""
    c = np.float32(float(q))
    cands = {np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))}
    best = None
    for v in sorted(cands):
        d = abs(Fraction(float(v)) - q)
        even = int(np.array(v, dtype=np.float32).view(np.uint32)) % 2 == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def test_gsa_closed_forms():
    # gsa = max|x| / (6 * 448) (commit 04cf8ca8, dsv4/layers/router.py, runtime-gsa paragraph).
    assert f32_hex(gsa_ref(2688.0)) == "3F800000"
    assert f32_hex(gsa_ref(4480.0)) == "3FD55555"
    assert gsa_ref(0.0) == 0.0
    rng = np.random.default_rng(3)
    amaxes = wl.bf16_to_f32(wl.bf16_bits(np.exp2(rng.uniform(-130, 120, 300)).astype(np.float32)))
    for a in amaxes:
        a = float(a)
        if a == 0.0:
            continue
        want = f32_nearest_exact(Fraction(a) / 2688)
        assert f32_hex(gsa_ref(a)) == f32_hex(want), a


@pytest.mark.parametrize("case", load_golden("quant_worked_examples.json")["cases"], ids=lambda c: c["name"])
def test_worked_examples(case):
    bits = bf16_exact(case["x"])[None, :]
    codes, scales, gsa = quantize_ref(bits, case["gsa_override"])
    assert f32_hex(gsa) == case["expect_gsa_hex"]
    assert scales[0].tolist() == hex_bytes(case["expect_scales_hex"]).tolist()
    assert codes[0].tolist() == hex_bytes(case["expect_codes_hex"]).tolist()
    # The exact-rational twin agrees on the same hand-worked case.
    c2, s2, g2 = quantize_exact_scalar(bits, case["gsa_override"])
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales) and f32_hex(g2) == f32_hex(gsa)


def test_static_scale_loses_magnitude_runtime_scale_does_not():
    # The failure the runtime gsa removed: a too-small static scale saturates the block scale.
    bits = bf16_exact([4480] + [0] * 15)[None, :]
    c_rt, s_rt, g_rt = quantize_ref(bits)
    c_st, s_st, g_st = quantize_ref(bits, gsa_override=1.0)
    v_rt = dequant_ref(c_rt, s_rt, g_rt)[0, 0]
    v_st = dequant_ref(c_st, s_st, g_st)[0, 0]
    assert v_st == 2688.0  # 40 % of the magnitude lost
    assert abs(v_rt - 4480.0) / 4480.0 < 1e-7


def _sweep_bits():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]  # finite patterns only


@pytest.mark.parametrize("gsa_hex,sbyte", [("3F800000", 0x7E), ("3FD55555", 0x58), ("3DA3D70A", 0x33),
                                             ("0A000000", 0x01), ("00000400", 0x7E)])
def test_element_rounding_exhaustive_bf16(gsa_hex, sbyte):
    """Every finite bf16 x against brute-force exact nearest, for several (gsa, S)."""
    gsa = np.array(int(gsa_hex, 16), dtype=np.uint32).view(np.float32)
    bits = _sweep_bits()
    x = wl.bf16_to_f32(bits).astype(np.float64)
    s = float(E4M3_GRID[sbyte])
    got = element_codes(x, s, gsa, bits >> 15)
    g = Fraction(float(gsa))
    sv = Fraction(s)
    for i in range(0, bits.size):
        mag = round_to_grid_exact(abs(Fraction(float(x[i]))) / (g * sv), E2M1_GRID)
        want = (int(bits[i]) >> 15) << 3 | mag
        assert int(got[i]) == want, (hex(int(bits[i])), int(got[i]), want)


@pytest.mark.parametrize("gsa_hex", ["3F800000", "3C23D70A", "00000200"])
def test_block_scale_rounding_sweep(gsa_hex):
    """Block maxima over every bf16 whose quotient lands in or near the E4M3 range."""
    gsa = np.array(int(gsa_hex, 16), dtype=np.uint32).view(np.float32)
    bits = _sweep_bits()
    bits = bits[bits < 0x8000]
    bmax = wl.bf16_to_f32(bits).astype(np.float64)
    q = bmax / (6.0 * float(gsa))
    keep = (q >= 2.0 ** -13) & (q <= 2.0 ** 10)
    bmax = bmax[keep]
    got = block_scale_bytes(bmax, gsa)
    den = 6 * Fraction(float(gsa))
    for v, b in zip(bmax, got):
        assert int(b) == round_to_grid_exact(Fraction(float(v)) / den, E4M3_GRID)


def _random_bits(rng, shape, kind):
    if kind == "normal":
        a = rng.standard_normal(shape).astype(np.float32)
    elif kind == "wide":
        a = (rng.standard_normal(shape) * np.exp2(rng.uniform(-40, 40, shape))).astype(np.float32)
    elif kind == "tiny":
        a = (rng.standard_normal(shape) * 2.0 ** -128).astype(np.float32)
    elif kind == "sparse":
        a = rng.standard_normal(shape).astype(np.float32) * (rng.random(shape) < 0.1)
        a[rng.random(shape) < 0.05] = -0.0
    else:
        raise ValueError(kind)
    return wl.bf16_bits(a)


@pytest.mark.parametrize("kind", ["normal", "wide", "tiny", "sparse"])
@pytest.mark.parametrize("override", [None, 1.0, 3e-3, 7e-39])
def test_vectorized_equals_exact_rational_twin(kind, override):
    kind_id = ["normal", "wide", "tiny", "sparse"].index(kind)
    rng = np.random.default_rng([11, kind_id, 0 if override is None else 1])
    bits = _random_bits(rng, (3, 48), kind)
    a = quantize_ref(bits, override)
    b = quantize_exact_scalar(bits, override)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and f32_hex(a[2]) == f32_hex(b[2])


@pytest.mark.parametrize("cfg", [1, 3])
def test_invariants_on_workloads(cfg):
    x = wl.make_x(cfg)
    codes, scales, gsa = quantize_ref(x)
    v = wl.bf16_to_f32(x).astype(np.float64)
    # x/gsa <= 2688 up to the single fp32 rounding of gsa (runtime-gsa paragraph, commit 04cf8ca8).
    assert np.max(np.abs(v)) / float(gsa) <= 2688.0 * (1 + 2.0 ** -23)
    assert scales.max() <= 0x7E  # never NaN, never above 448
    # Dequantization error per element is at most half an E2M1 step of its block (or saturation).
    deq = dequant_ref(codes, scales, gsa)
    step = np.repeat(E4M3_GRID[scales.astype(int)], 16, axis=1) * float(gsa)
    err = np.abs(deq - v)
    assert np.all(err <= 1.0 * step)


def test_round_trip_of_on_grid_tensor():
    """x = val(q) * val(S) with every block's max code 6 and one block at S = 448: q, S come back."""
    rng = np.random.default_rng(5)
    rows, d = 64, 7168
    nb = d // 16
    sbytes = rng.integers(1, 0x7F, size=(rows, nb)).astype(np.uint8)
    sbytes[0, 0] = 0x7E
    mags = rng.integers(0, 8, size=(rows, nb, 16))
    lead = rng.integers(0, 16, size=(rows, nb))
    np.put_along_axis(mags, lead[:, :, None], 7, axis=2)
    signs = rng.integers(0, 2, size=(rows, nb, 16))
    codes = (signs << 3 | mags).astype(np.uint8).reshape(rows, d)
    x = dequant_ref(pack_codes(codes), sbytes, 1.0)  # code 0x8 gives -0.0
    bits = wl.bf16_bits(x.astype(np.float32))
    assert np.array_equal(wl.bf16_to_f32(bits).astype(np.float64), x)
    c2, s2, g2 = quantize_ref(bits)
    assert float(g2) == 1.0
    assert np.array_equal(s2, sbytes)
    assert np.array_equal(c2, pack_codes(codes))


def test_zero_tensor_and_negative_zero():
    bits = np.zeros((2, 32), dtype=np.uint16)
    bits[1, 3] = 0x8000
    codes, scales, gsa = quantize_ref(bits)
    assert gsa == 0.0 and scales.max() == 0
    u = unpack_codes(codes)
    assert u[1, 3] == 0x8 and u.sum() == 0x8


def test_packing_low_nibble_is_even_element():
    codes = np.array([[1, 2, 3, 4, 15, 0, 8, 7]], dtype=np.uint8)
    assert pack_codes(codes)[0].tolist() == [0x21, 0x43, 0x0F, 0x78]
    assert np.array_equal(unpack_codes(pack_codes(codes)), codes)
