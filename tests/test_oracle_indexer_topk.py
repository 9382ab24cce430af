"""Pins of the lightning indexer and Top-k of the oracle.

Indexer: "DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" 4.1 (a cheap
score I_{t,s} per query and history entry, few heads, FP8), with the score
form sum_h w_h ReLU(q_h . k_s).  Top-k: same page, 4.2, S_t = TopK(I_t, k)."""

from fractions import Fraction

import numpy as np

from oracle import codecs, dsa


def test_indexer_special_cases():
    rng = np.random.default_rng(0)
    q, k = rng.standard_normal((4, 16)), rng.standard_normal((50, 16))
    assert not dsa.indexer_scores(q, np.zeros(4), k).any()
    # keys anti-aligned with every head: all dots negative -> zero score
    qq = np.abs(q)
    assert not dsa.indexer_scores(qq, np.ones(4), -np.abs(k)).any()
    # one head, unit weight: plain ReLU of the dot product
    s1 = dsa.indexer_scores(q[:1], np.ones(1), k)
    assert np.array_equal(s1, np.maximum(k @ q[0], 0.0))
    # heads add linearly in w
    w = rng.standard_normal(4)
    tot = sum(w[h] * dsa.indexer_scores(q[h:h + 1], np.ones(1), k) for h in range(4))
    assert np.allclose(dsa.indexer_scores(q, w, k), tot, atol=1e-12)


def test_indexer_exact_on_fp8_values():
    """On fp8 values the fp64 oracle is exact up to the final multiplies: every
    e4m3fn value is a multiple of 2^-9, products are multiples of 2^-18 and a
    128-term dot product fits fp64's 53 bits.  Checked with exact rationals."""
    rng = np.random.default_rng(1)
    qc = codecs.fp8_encode(rng.standard_normal((3, 128)) * 60)
    kc = codecs.fp8_encode(rng.standard_normal((20, 128)) * 60)
    q, k = codecs.fp8_decode(qc), codecs.fp8_decode(kc)
    w = np.array([0.5, -1.25, 2.0])  # dyadic, so the weighted sum is exact too
    got = dsa.indexer_scores(q, w, k)
    for j in range(20):
        ex = Fraction(0)
        for h in range(3):
            d = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q[h], k[j]))
            ex += Fraction(float(w[h])) * max(d, Fraction(0))
        assert Fraction(float(got[j])) == ex


def test_topk_invariants():
    rng = np.random.default_rng(2)
    for n, k in [(1000, 64), (300, 512), (0, 8), (64, 64), (65, 64)]:
        sc = rng.standard_normal(n)
        idx, vals = dsa.topk(sc, k)
        sel = idx[idx >= 0]
        assert len(idx) == k and len(sel) == min(k, n)
        assert np.all(np.diff(sel) > 0) and np.all(sel < n)
        assert np.all(idx[len(sel):] == -1)
        if 0 < len(sel) < n:
            rest = np.setdiff1d(np.arange(n), sel)
            assert sc[sel].min() >= sc[rest].max()


def test_topk_ties_prefer_lower_index():
    sc = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 2.0, 0.5])
    idx, _ = dsa.topk(sc, 4)
    assert idx.tolist() == [1, 2, 3, 4]
    idx, _ = dsa.topk(np.zeros(10), 3)
    assert idx.tolist() == [0, 1, 2]


def test_topk_against_brute_force():
    rng = np.random.default_rng(3)
    sc = np.round(rng.standard_normal(40), 1)  # many ties
    k = 11
    brute = sorted(range(40), key=lambda j: (-sc[j], j))[:k]
    idx, _ = dsa.topk(sc, k)
    assert idx.tolist() == sorted(brute)
