"""Pins of the RoPE reading: identity, isometry, relative property, hand values."""
import numpy as np

from oracle.rope import rope, rope_freqs


def test_frequencies_hand_values():
    assert np.allclose(rope_freqs(4, 100.0), [1.0, 0.1], rtol=0, atol=1e-15)
    w = rope_freqs(128, 1e6)
    assert w[0] == 1.0 and abs(w[64 - 1] - 1e6 ** (-126 / 128)) < 1e-20


def test_hand_rotation_pairs_i_with_i_plus_half():
    # d = 4, theta = 100: pair (0, 2) turns at 1 rad/pos, pair (1, 3) at 0.1.
    out = rope(np.array([1.0, 0.0, 0.0, 0.0]), 1.0, 100.0)
    assert np.allclose(out, [np.cos(1.0), 0.0, np.sin(1.0), 0.0], atol=1e-15)
    out = rope(np.array([0.0, 1.0, 0.0, 0.0]), 2.0, 100.0)
    assert np.allclose(out, [0.0, np.cos(0.2), 0.0, np.sin(0.2)], atol=1e-15)
    out = rope(np.array([0.0, 0.0, 1.0, 0.0]), 1.0, 100.0)
    assert np.allclose(out, [-np.sin(1.0), 0.0, np.cos(1.0), 0.0], atol=1e-15)


def test_two_dims_is_complex_multiplication():
    r = np.random.default_rng(1)
    x = r.standard_normal(2)
    for p in [0.0, 1.0, 7.0, 1234.0]:
        z = complex(x[0], x[1]) * np.exp(1j * p)
        assert np.allclose(rope(x, p, 10.0), [z.real, z.imag], atol=1e-12)


def test_position_zero_is_identity_and_norm_is_kept():
    r = np.random.default_rng(2)
    x = r.standard_normal((5, 64))
    assert np.array_equal(rope(x, np.zeros(5), 1e4), x)
    y = rope(x, np.arange(5) * 1000.0, 1e4)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_relative_position_property():
    r = np.random.default_rng(3)
    q, k = r.standard_normal(128), r.standard_normal(128)
    for a, b in [(10.0, 3.0), (4096.0, 17.0), (33000.0, 32999.0)]:
        lhs = rope(q, a, 1e6) @ rope(k, b, 1e6)
        rhs = rope(q, a - b, 1e6) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))
