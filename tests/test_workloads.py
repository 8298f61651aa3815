"""The seeded input generators: shapes, determinism and the bf16 rounding of samples."""

import numpy as np

from nvfp4_block_scaled_06_amd import workloads as wl


def test_bf16_rounding_is_nearest_even():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0); 1 + 3*2^-8 rounds up to 1 + 2^-6.
    assert wl.bf16_to_f32(wl.bf16_bits(a)).tolist()[:4] == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]


def test_shapes_and_determinism_small_configs():
    for cfg in (1, 3):
        c = wl.CONFIGS[cfg]
        x, w, b = wl.make_x(cfg), wl.make_w(cfg), wl.make_bias(cfg)
        assert x.shape == (c.T, c.D) and x.dtype == np.uint16
        assert w.shape == (c.E, c.D) and b.shape == (c.E,) and b.dtype == np.float32
        assert np.array_equal(x, wl.make_x(cfg)) and np.array_equal(w, wl.make_w(cfg))
        assert np.all(np.abs(b) <= c.bias_half_width)
    assert not np.array_equal(wl.make_w(2, 0), wl.make_w(2, 1))
    assert wl.make_x(2, 5).shape == (1, 7168)


def test_outlier_channels_in_batched_decode():
    v = np.abs(wl.bf16_to_f32(wl.make_x(3)))
    col = v.max(axis=0)
    assert (col > 40).sum() >= 60  # about 72 channels scaled by 50
    assert np.median(col) < 5


def test_sample_rows():
    r = wl.sample_rows(8192, 64)
    assert r[0] == 0 and r[-1] == 8191 and len(r) == 64 and np.all(np.diff(r) > 0)
