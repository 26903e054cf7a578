"""Pins for the oracle's building blocks (CPU only).

Each test fixes a value or property the definitions fix: worked values,
closed forms, invariants and special cases that reduce to something simpler.
"""

import cmath
import math

import numpy as np
import pytest

from oracle import decoder as D


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_worked_example():
    x = np.array([1.0, 2.0, 3.0, 4.0])
    y = D.rmsnorm(x, np.ones(4), 0.0)
    # mean of squares is 7.5
    np.testing.assert_allclose(y, x / math.sqrt(7.5), rtol=0, atol=1e-15)
    np.testing.assert_allclose(y, [0.365148371670111, 0.730296743340221,
                                   1.095445115010332, 1.460593486680443], atol=1e-12)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 33))
    y = D.rmsnorm(x, np.ones(33), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, atol=1e-13)
    np.testing.assert_allclose(D.rmsnorm(7.3 * x, np.ones(33), 0.0), y, atol=1e-13)
    # no centring: a constant vector maps to +-1, not 0
    np.testing.assert_allclose(D.rmsnorm(np.full(8, -3.0), np.ones(8), 0.0), -1.0, atol=1e-15)


def test_rmsnorm_gain_and_eps():
    x = np.array([3.0, 4.0])  # mean square 12.5
    g = np.array([2.0, -0.5])
    eps = 1e-5
    np.testing.assert_allclose(D.rmsnorm(x, g, eps), g * x / math.sqrt(12.5 + eps), atol=1e-15)


# ------------------------------------------------------------------ RoPE

def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).standard_normal((3, 64))
    np.testing.assert_array_equal(D.rope(x, 0, 1e4), x)


def test_rope_dh2_position1():
    y = D.rope(np.array([1.0, 0.0]), 1, 1e4)
    np.testing.assert_allclose(y, [0.5403023058681398, 0.8414709848078965], atol=1e-15)


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(128)
    y = D.rope(x, 777, 1e4)
    np.testing.assert_allclose(np.hypot(y[0::2], y[1::2]), np.hypot(x[0::2], x[1::2]), atol=1e-12)


def test_rope_relative_position_property():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    a = D.rope(q, 10, 1e4) @ D.rope(k, 3, 1e4)
    b = D.rope(q, 107, 1e4) @ D.rope(k, 100, 1e4)
    np.testing.assert_allclose(a, b, atol=1e-10)


def test_rope_composition():
    x = np.random.default_rng(4).standard_normal(64)
    np.testing.assert_allclose(D.rope(D.rope(x, 5, 1e4), 9, 1e4), D.rope(x, 14, 1e4), atol=1e-12)


def test_rope_matches_complex_rotation_of_adjacent_pairs():
    """Adjacent pair (x_2i, x_2i+1) as a complex number times e^{i p theta^(-2i/dh)}."""
    rng = np.random.default_rng(5)
    dh, p, theta = 16, 37, 1e4
    x = rng.standard_normal(dh)
    y = D.rope(x, p, theta)
    for i in range(dh // 2):
        z = complex(x[2 * i], x[2 * i + 1]) * cmath.exp(1j * p * theta ** (-2.0 * i / dh))
        assert abs(y[2 * i] - z.real) < 1e-12 and abs(y[2 * i + 1] - z.imag) < 1e-12


def test_rope_frequencies():
    phi = D.rope_angles(1, 8, 1e4)
    np.testing.assert_allclose(phi, [1.0, 0.1, 0.01, 0.001], rtol=1e-14)


# ------------------------------------------------------------------ softmax / silu

def test_softmax_properties():
    rng = np.random.default_rng(6)
    z = rng.standard_normal((4, 17)) * 10
    a = D.softmax(z)
    np.testing.assert_allclose(a.sum(-1), 1.0, atol=1e-14)
    np.testing.assert_allclose(D.softmax(z + 123.0), a, atol=1e-14)
    np.testing.assert_array_equal(D.softmax(np.array([3.7])), [1.0])
    np.testing.assert_allclose(D.softmax(np.array([0.0, math.log(3.0)])), [0.25, 0.75], atol=1e-15)


def test_silu_values():
    assert D.silu(np.array(0.0)) == 0.0
    assert abs(D.silu(np.array(1.0)) - 0.7310585786300049) < 1e-15
    assert abs(D.silu(np.array(40.0)) - 40.0) < 1e-12
    assert abs(D.silu(np.array(-40.0))) < 1e-15
    assert abs(D.silu(np.array(-1.0)) - (-0.2689414213699951)) < 1e-15


# ------------------------------------------------------------------ attention

def test_single_key_returns_value():
    rng = np.random.default_rng(7)
    q, K, V = rng.standard_normal(64), rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    np.testing.assert_array_equal(D.attend(q, K, V), V[0])


def test_equal_keys_average_values():
    rng = np.random.default_rng(8)
    q = rng.standard_normal(32)
    K = np.tile(rng.standard_normal(32), (5, 1))
    V = rng.standard_normal((5, 32))
    np.testing.assert_allclose(D.attend(q, K, V), V.mean(0), atol=1e-14)


def test_attention_scale_and_weights():
    dh = 4
    q = np.array([1.0, 0.0, 0.0, 0.0])
    K = np.array([[0.0, 0, 0, 0], [2.0 * math.log(3.0), 0, 0, 0]])  # scores 0 and log 3
    V = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
    np.testing.assert_allclose(D.attend(q, K, V), [0.25, 0.75, 0, 0], atol=1e-15)
    assert math.sqrt(dh) == 2.0


# ------------------------------------------------------------------ stored matrices

@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_matvec_with_scales_matches_loops(fmt):
    from oracle import codecs
    rng = np.random.default_rng(9)
    rows, cols, B = 7, 11, 3
    if fmt == "bf16":
        codes = codecs.bf16_encode(rng.standard_normal((rows, cols)) * 0.1)
        scale = None
    else:
        codes = rng.integers(0, 256, (rows, cols)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x10  # no NaN codes
        scale = rng.uniform(0.001, 0.01, rows).astype(np.float32)
    m = D.Matrix(rows, cols, fmt, codes=codes, scale=scale, chunk_rows=3)
    X = rng.standard_normal((B, cols))
    Y = m.matvec(X)
    for b in range(B):
        for r in range(rows):
            acc = 0.0
            for c in range(cols):
                w = codecs.decode(codes[r:r + 1, c:c + 1], fmt)[0, 0]
                acc += w * X[b, c]
            if scale is not None:
                acc *= float(scale[r])
            assert abs(Y[b, r] - acc) < 1e-12 * max(1.0, abs(acc))


def test_kv_bytes_per_token_formula():
    assert D.kv_bytes_per_token(80, 8, 128, 2) == 327680
