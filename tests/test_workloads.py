"""The seeded generators: deterministic, right shapes, right distributions."""
import numpy as np

from workloads import CONFIGS, bf16_bits_from_f32, f32_from_bf16_bits, make_activation, make_layer


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e38], dtype=np.float32)
    b = bf16_bits_from_f32(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    np.testing.assert_array_equal(b[:4], np.array([0x3F80, 0x3F80, 0x3F82, 0xBF80], dtype=np.uint16))
    assert abs(f32_from_bf16_bits(b[4:])[0] / 3.0e38 - 1) < 2 ** -8


def test_deterministic_and_seed_sensitive():
    a = make_activation("heavy", 8, 512, seed=0)
    b = make_activation("heavy", 8, 512, seed=0)
    c = make_activation("heavy", 8, 512, seed=1)
    np.testing.assert_array_equal(a, b)
    assert np.any(a != c)


def test_tiny_config_shapes_and_distribution():
    L = make_layer(256, 512, 512, "heavy", seed=0)
    assert L.X.shape == (256, 512) and L.W.shape == (512, 512)
    assert L.LA.shape == (512, 64) and L.LB.shape == (64, 512)
    x = f32_from_bf16_bits(L.X).astype(np.float64)
    col_rms = np.sqrt((x * x).mean(axis=0))
    # 1% of channels (5 of 512) boosted x20: the largest columns stand out
    assert np.sort(col_rms)[-5:].min() > 5 * np.median(col_rms)
    w = f32_from_bf16_bits(L.W).astype(np.float64)
    assert abs(w.std() * np.sqrt(512) - 1) < 0.02
    assert abs(f32_from_bf16_bits(L.LA).std() / 0.02 - 1) < 0.05


def test_gelu_activation_is_skewed():
    x = f32_from_bf16_bits(make_activation("gelu", 64, 1024, seed=0)).astype(np.float64)
    # GELU(z) >= -0.17, so per channel the negative side is bounded by 0.17 c[k]
    assert x.mean() > 0 and x.min() > -0.2 * x.max()


def test_config_table():
    assert CONFIGS["mlp_up"] == [(4096, 3072, 12288, "heavy")]
    assert [l[2] for l in CONFIGS["block"]] == [9216, 3072, 12288, 3072]
