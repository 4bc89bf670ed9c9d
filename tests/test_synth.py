"""The seeded input generators: determinism and the documented distributions."""
import numpy as np

import synth


def test_bf16_rounding_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.005859375, 1.0029296875, -3.14159, 0.0], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    back = synth.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert back[1] == 1.0
    # 1 + 1.5*2^-8 rounds up to 1 + 2^-7
    assert back[2] == np.float32(1.0078125)
    assert back[3] == 1.0
    assert abs(back[4] - vals[4]) <= 2 ** -8 * abs(vals[4])
    assert bits[5] == 0


def test_make_linear_is_deterministic():
    a = synth.make_linear("single-1024", 0, 1, seed=0)
    b = synth.make_linear("single-1024", 0, 1, seed=0)
    c = synth.make_linear("single-1024", 0, 1, seed=1)
    for key in ("codes", "scales", "x"):
        np.testing.assert_array_equal(a[key], b[key])
    assert not np.array_equal(a["codes"], c["codes"])


def test_uniform_recipe_ranges():
    d = synth.make_linear("single-1024", 0, 4, seed=0)
    assert d["codes"].shape == (1024, 1024) and d["scales"].shape == (1024, 8)
    assert abs(d["codes"].mean() - 127.5) < 1.0
    s = synth.bf16_bits_to_f32(d["scales"])
    assert s.min() >= 0.000999 and s.max() <= 0.01001
    x = synth.bf16_bits_to_f32(d["x"])
    assert abs(x.mean()) < 0.1 and abs(x.std() - 1.0) < 0.1


def test_gptq_like_codes_are_nearest_grid_levels():
    rng = np.random.default_rng(3)
    codes, scales = synth.gptq_like(64, 512, rng)
    rng2 = np.random.default_rng(3)
    w = rng2.normal(0.0, 0.02, size=(64, 512)).astype(np.float32).astype(np.float64)
    s = np.repeat(synth.bf16_bits_to_f32(scales).astype(np.float64), 128, axis=1)
    level = s * (codes.astype(np.float64) - 127.5)
    # nearest level of the 8-bit grid (clamped at the ends)
    assert np.all(np.abs(w - level) <= s / 2 + 1e-12 + np.where((codes == 0) | (codes == 255), s, 0))
    assert codes.min() >= 0 and codes.max() <= 255


def test_outlier_channels():
    k = 4096
    x = synth.bf16_bits_to_f32(synth.activations(8, k, np.random.default_rng(0), outliers=True,
                                                 outlier_rng=np.random.default_rng(1)))
    col_std = x.std(axis=0)
    assert int((col_std > 4).sum()) == round(0.01 * k)
