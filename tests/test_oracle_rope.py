"""Pins of the oracle's rotary embedding.

The pages fix the relative-position identity R_m R_n^T = R_(m-n) and the
inverse R_m^{-1} ("DeepSeek V4 稀疏注意力完全解剖", 深潜: 为什么必须做 Inverse
RoPE).  The pair layout and frequency schedule are a convention (parity
unpinned for the layout); these tests pin the identities, orthogonality and
agreement with the complex-number form of a 2-D rotation."""

import numpy as np
import pytest

from oracle import dsa

R, BASE, D = 16, 10000.0, 40


def test_zero_position_is_identity_and_other_dims_untouched():
    x = np.random.default_rng(0).standard_normal((5, D))
    assert np.array_equal(dsa.rope_rotate(x, np.zeros(5), R, BASE), x)
    y = dsa.rope_rotate(x, np.arange(5) * 1000.0, R, BASE)
    assert np.array_equal(y[:, :D - R], x[:, :D - R])
    assert np.array_equal(dsa.rope_rotate(x, 123.0, 0, BASE), x)


def test_orthogonal():
    x = np.random.default_rng(1).standard_normal((7, D))
    y = dsa.rope_rotate(x, np.array([0, 1, 17, 4096, 65535, 1048575, 3]), R, BASE)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


@pytest.mark.parametrize("m,n", [(5, 3), (1048575, 1048447), (0, 77), (131071, 126976)])
def test_relative_identity(m, n):
    rng = np.random.default_rng(m + n)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    # R_m R_n^{-1} = R_(m-n)
    assert np.allclose(dsa.rope_rotate(dsa.rope_inverse(k, n, R, BASE), m, R, BASE),
                       dsa.rope_rotate(k, m - n, R, BASE), atol=1e-9)
    # (R_m q) . (R_n k) depends only on n - m
    lhs = dsa.rope_rotate(q, m, R, BASE) @ dsa.rope_rotate(k, n, R, BASE)
    rhs = q @ dsa.rope_rotate(k, n - m, R, BASE)
    assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(rhs))


def test_matches_complex_rotation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(D)
    p = 98765.0
    z = x[D - R::2] + 1j * x[D - R + 1::2]
    theta = BASE ** (-np.arange(R // 2) * 2.0 / R)
    zr = z * np.exp(1j * p * theta)
    y = dsa.rope_rotate(x, p, R, BASE)
    assert np.allclose(y[D - R::2], zr.real, atol=1e-12)
    assert np.allclose(y[D - R + 1::2], zr.imag, atol=1e-12)


def test_inverse():
    x = np.random.default_rng(4).standard_normal((3, D))
    pos = np.array([9.0, 100000.0, 1048575.0])
    assert np.allclose(dsa.rope_inverse(dsa.rope_rotate(x, pos, R, BASE), pos, R, BASE), x,
                       atol=1e-12)
