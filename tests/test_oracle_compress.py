"""Pins of the oracle compressor: special cases with closed forms, a
library formulation of the strided weighted sum, RMSNorm and the fp8
quantisation of an entry.

Compressor per "DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" 5.2 and
"DeepSeek V4 稀疏注意力完全解剖" 机制二: entry j = weighted sum of raw tokens
s j .. s j + S - 1 (c4a: S=8, s=4; c128a: S=s=128)."""

import numpy as np
import pytest
from numpy.lib.stride_tricks import sliding_window_view

from oracle import codecs, dsa


def _raw(L, D, seed=0):
    return np.random.default_rng(seed).standard_normal((L, D))


@pytest.mark.parametrize("s,S", [(4, 8), (128, 128)])
def test_uniform_logits_give_the_mean(s, S):
    X = _raw(4 * S, 12)
    n = dsa.n_complete(len(X), s, S)
    c = dsa.compress_range(lambda p: X[p], np.zeros((n, S)), 0, n, s, S, r=0, base=1.0)
    for j in range(n):
        assert np.allclose(c[j], X[s * j:s * j + S].mean(axis=0), atol=1e-14)


def test_one_hot_logits_copy_one_token():
    s, S = 4, 8
    X = _raw(64, 10)
    for i in range(S):
        lg = np.full((1, S), -1000.0)
        lg[0, i] = 0.0
        c = dsa.compress_range(lambda p: X[p], lg, 5, 1, s, S, r=0, base=1.0)[0]
        assert np.array_equal(c, X[s * 5 + i])


@pytest.mark.parametrize("s,S", [(4, 8), (128, 128), (3, 5)])
def test_strided_weighted_sum_matches_einsum(s, S):
    L, D = 3 * S + 11, 6
    X = _raw(L, D, 1)
    n = dsa.n_complete(L, s, S)
    lg = np.random.default_rng(2).standard_normal((n, S))
    c = dsa.compress_range(lambda p: X[p], lg, 0, n, s, S, r=0, base=1.0)
    win = sliding_window_view(X, S, axis=0)[::s][:n]          # [n, D, S]
    wts = np.exp(lg) / np.exp(lg).sum(axis=1, keepdims=True)
    ref = np.einsum("nds,ns->nd", win, wts)
    assert np.allclose(c, ref, atol=1e-13)


def test_rotation_at_first_token_position():
    s, S, r, base = 4, 8, 4, 10000.0
    X = _raw(40, 8, 3)
    lg = np.random.default_rng(4).standard_normal((1, S))
    c = dsa.compress_range(lambda p: X[p], lg, 3, 1, s, S, r=r, base=base, pos_offset=100)[0]
    plain = dsa.compress_range(lambda p: X[p], lg, 3, 1, s, S, r=0, base=base)[0]
    assert np.allclose(c, dsa.rope_rotate(plain, s * 3 + 100, r, base), atol=1e-13)
    assert np.array_equal(c[:8 - r], plain[:8 - r])


def test_rmsnorm_optional():
    s, S = 4, 8
    X = _raw(16, 32, 5)
    lg = np.random.default_rng(6).standard_normal((1, S))
    c = dsa.compress_range(lambda p: X[p], lg, 0, 1, s, S, r=0, base=1.0,
                           gamma=np.ones(32), eps=0.0)[0]
    assert abs(np.sqrt(np.mean(c ** 2)) - 1.0) < 1e-12
    g = np.linspace(0.5, 2.0, 32)
    c2 = dsa.compress_range(lambda p: X[p], lg, 0, 1, s, S, r=0, base=1.0, gamma=g, eps=0.0)[0]
    assert np.allclose(c2, g * c, atol=1e-13)


def test_fp8_entry_quantisation():
    c = np.random.default_rng(7).standard_normal(128) * 3.0
    codes, sigma = dsa.quantize_fp8_entry(c)
    assert sigma == float(np.float32(np.max(np.abs(c)) / 448.0))
    deq = codecs.fp8_decode(codes)
    # the largest element lands on (or next to) the top of the grid
    assert np.max(np.abs(deq)) >= 416.0
    # round to nearest: error at most half a grid step of e4m3fn (2^-4 relative
    # in a binade, 2^-10 absolute in the subnormal range), in code units
    x = c / sigma
    step = np.where(np.abs(x) < 2 ** -6, 2.0 ** -9,
                    2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 1e-300))) - 3))
    assert np.all(np.abs(deq - x) <= step / 2 + 1e-12)
    z, s0 = dsa.quantize_fp8_entry(np.zeros(16))
    assert s0 == 0.0 and not z.any()
