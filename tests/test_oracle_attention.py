"""Pins of the oracle attention step and of whole-layer invariances.

* Special cases with closed forms (one vector, zero query, empty set).
* Dense equivalence against torch's scaled_dot_product_attention (CPU, fp64).
* Translation invariance of the output after R_m^{-1} ("DeepSeek V4 稀疏注意力
  完全解剖", 深潜: 为什么必须做 Inverse RoPE): shifting every position by a
  constant leaves the output unchanged; without the inverse rotation it
  does not (negative control).
* c128a with k >= n_vis is dense attention over every visible entry plus the
  window (same page, 机制三).
* Chunk invariance: a prefill split into chunks of any size (the compressor
  state carries the last S raw tokens across the boundary, [P2] 设计 2)
  equals one pass.
"""

import numpy as np
import pytest
import torch

from oracle import dsa
from oracle.layer import Geometry, SeqState, layer_chunk

R, BASE = 8, 10000.0


def test_single_vector_and_zero_query():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1, 16))
    q = rng.standard_normal((3, 16))
    out, lse = dsa.sparse_attention(q, v, 77, R, BASE, 0.25)
    assert np.allclose(out, dsa.rope_inverse(np.repeat(v, 3, 0), 77, R, BASE), atol=1e-14)
    assert np.allclose(lse, 0.25 * (q @ v[0]), atol=1e-14)
    V = rng.standard_normal((9, 16))
    out, lse = dsa.sparse_attention(np.zeros((2, 16)), V, 5, R, BASE, 0.25)
    assert np.allclose(out, dsa.rope_inverse(np.repeat(V.mean(0, keepdims=True), 2, 0), 5, R,
                                             BASE), atol=1e-14)
    assert np.allclose(lse, np.log(9.0))
    out, lse = dsa.sparse_attention(q, np.zeros((0, 16)), 5, R, BASE, 0.25)
    assert not out.any() and np.all(np.isneginf(lse))


def test_matches_torch_sdpa():
    rng = np.random.default_rng(1)
    H, A, D = 8, 37, 32
    q, V = rng.standard_normal((H, D)), rng.standard_normal((A, D))
    tau = 1 / np.sqrt(D)
    out, lse = dsa.sparse_attention(q, V, 0, 0, BASE, tau)
    tq = torch.from_numpy(q)[None, :, None, :]          # [1, H, 1, D]
    tv = torch.from_numpy(V)[None, None].expand(1, H, A, D)  # K = V shared by heads
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tv, tv, scale=tau)[0, :, 0]
    assert np.allclose(out, ref.numpy(), atol=1e-12)
    assert np.allclose(lse, torch.logsumexp(torch.from_numpy(tau * q @ V.T), 1).numpy(),
                       atol=1e-12)


def _geom(**kw):
    d = dict(s=4, S=8, D=24, r=R, Di=16, r_idx=0, H=4, Hi=3, k=6, W=10,
             main_dtype="f64", idx_dtype="f64")
    d.update(kw)
    return Geometry(**d)


def _fresh_state(g, E_cap, W_cap=None):
    return SeqState(main_cache=np.zeros((E_cap, g.D)), idx_cache=np.zeros((E_cap, g.Di)),
                    idx_scale=np.ones(E_cap), main_ring=np.zeros((g.S, g.D)),
                    idx_ring=np.zeros((g.S, g.Di)),
                    win_ring=np.zeros((W_cap or g.W, g.D)))


def _seq(g, L, seed):
    rng = np.random.default_rng(seed)
    n = dsa.n_complete(L, g.s, g.S)
    return dict(X=rng.standard_normal((L, g.D)), KX=rng.standard_normal((L, g.Di)),
                LM=rng.standard_normal((n, g.S)), LI=rng.standard_normal((n, g.S)),
                Q=rng.standard_normal((L, g.H, g.D)), QI=rng.standard_normal((L, g.Hi, g.Di)),
                WT=rng.standard_normal((L, g.Hi)))


def _run_chunks(g, d, L, sizes, W_cap=None):
    st = _fresh_state(g, dsa.n_slots(L, g.s), W_cap)
    outs, lses, idxs = [], [], []
    p = 0
    for T in sizes:
        j0, j1 = dsa.n_complete(p, g.s, g.S), dsa.n_complete(p + T, g.s, g.S)
        o, l, ix = layer_chunk(g, st, p, d["X"][p:p + T], d["KX"][p:p + T], d["LM"][j0:j1],
                               d["LI"][j0:j1], d["Q"][p:p + T], d["QI"][p:p + T],
                               d["WT"][p:p + T])
        outs.append(o), lses.append(l), idxs.append(ix)
        p += T
    assert p == L
    return np.concatenate(outs), np.concatenate(lses), np.concatenate(idxs), st


@pytest.mark.parametrize("sizes", [[1] * 60, [7, 13, 5, 35], [3, 57], [29, 31]])
def test_chunk_invariance(sizes):
    g = _geom()
    L = sum(sizes)
    d = _seq(g, L, 5)
    ref = _run_chunks(g, d, L, [L])
    got = _run_chunks(g, d, L, sizes)
    for a, b in zip(ref[:3], got[:3]):
        assert np.array_equal(a, b)
    assert np.array_equal(ref[3].main_cache, got[3].main_cache)


def test_chunk_invariance_c128a_and_ring_wider_than_window():
    g = _geom(s=16, S=16, Hi=0, k=64, W=10)
    L = 100
    d = _seq(g, L, 6)
    ref = _run_chunks(g, d, L, [L], W_cap=12)
    got = _run_chunks(g, d, L, [17, 1, 1, 40, 41], W_cap=12)
    for a, b in zip(ref[:3], got[:3]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("shift", [1, 1000, 123457, 1048575])
def test_translation_invariance(shift):
    g0 = _geom()
    g1 = _geom(pos_offset=shift)
    L = 48
    d = _seq(g0, L, 7)
    o0, l0, i0, _ = _run_chunks(g0, d, L, [L])
    o1, l1, i1, _ = _run_chunks(g1, d, L, [L])
    assert np.array_equal(i0, i1)          # the indexer keys carry no rotation
    assert np.max(np.abs(o0 - o1)) < 1e-9
    fin = np.isfinite(l0)
    assert np.array_equal(fin, np.isfinite(l1)) and not fin[0].any()  # m=0: empty set
    assert np.max(np.abs(l0[fin] - l1[fin])) < 1e-9


def test_without_inverse_rope_output_is_not_translation_invariant():
    rng = np.random.default_rng(8)
    q, V = rng.standard_normal((2, 16)), rng.standard_normal((5, 16))
    pos = np.array([3, 9, 11, 14, 15])
    outs = []
    for c in (0, 1000):
        vr = dsa.rope_rotate(V, pos + c, R, BASE)
        qr = dsa.rope_rotate(q, 16 + c, R, BASE)
        o, _ = dsa.sparse_attention(qr, vr, 0, R, BASE, 0.25)  # position 0: no inverse
        outs.append(o)
    assert np.max(np.abs(outs[0] - outs[1])) > 1e-3


def test_c128a_full_selection_is_dense_attention():
    g = _geom(s=16, S=16, Hi=0, k=64, W=10)
    L = 90
    d = _seq(g, L, 9)
    out, lse, idx, st = _run_chunks(g, d, L, [L])
    for t in [0, 15, 16, 31, 32, 60, 89]:
        nv = dsa.n_vis(t, g.s, g.S)
        assert idx[t][:nv].tolist() == list(range(nv)) and np.all(idx[t][nv:] == -1)
        ents = st.main_cache[:nv]
        win = dsa.rope_rotate(d["X"][max(0, t - g.W):t], np.arange(max(0, t - g.W), t), g.r,
                              g.base)
        allv = np.concatenate([ents, win])
        if len(allv) == 0:
            assert not out[t].any()
            continue
        qr = dsa.rope_rotate(d["Q"][t], t, g.r, g.base)
        tq = torch.from_numpy(qr)[None, :, None, :]
        tv = torch.from_numpy(allv)[None, None].expand(1, g.H, len(allv), g.D)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tv, tv, scale=g.tau)[0, :, 0]
        ref = dsa.rope_inverse(ref.numpy(), t, g.r, g.base)
        assert np.allclose(out[t], ref, atol=1e-12)


def test_softmax_scale_is_one_over_sqrt_d():
    # "DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" 2: softmax(Q K^T / sqrt(d)) V
    assert _geom(D=512).tau == 1 / np.sqrt(512)
    assert _geom(D=128, scale=0.5).tau == 0.5


def test_fp8_output_is_nearest_code_per_head():
    """The fp8 output of each head is, element by element, the nearest of the
    255 finite e4m3fn values times the head's scale max|o| / 448 (brute force
    over every code), and an all-zero head gives scale 0 and zero codes."""
    from oracle import codecs
    rng = np.random.default_rng(11)
    out = rng.standard_normal((4, 40)) * np.array([[0.02], [1.0], [37.0], [0.0]])
    codes, sig = dsa.quantize_fp8_heads(out)
    assert codes.shape == out.shape and codes.dtype == np.uint8 and sig.shape == (4,)
    grid = codecs.fp8_decode(np.arange(256, dtype=np.uint8))
    finite = np.isfinite(grid)
    for h in range(3):
        assert sig[h] == float(np.float32(np.abs(out[h]).max() / 448.0))
        for d in range(out.shape[1]):
            x = out[h, d] / sig[h]
            dist = np.where(finite, np.abs(grid - x), np.inf)
            best = np.flatnonzero(dist == dist.min())
            assert codes[h, d] in best, (h, d, x)
        # the largest magnitude maps to the top of the grid
        assert np.abs(codecs.fp8_decode(codes[h])).max() == 448.0
    assert sig[3] == 0.0 and not codes[3].any()


def test_q_norm_is_rms_norm():
    """The Q-norm reading (RMSNorm of each head over its D dims) against
    torch's rms_norm in float64, and its closed form with gamma = 1."""
    import torch
    from oracle import dsa
    rng = np.random.default_rng(11)
    q = rng.standard_normal((5, 64, 32)) * 3.0
    gamma = 1.0 + 0.5 * rng.standard_normal(32)
    eps = 1e-6
    ref = torch.nn.functional.rms_norm(torch.from_numpy(q), (32,), torch.from_numpy(gamma),
                                       eps=eps).numpy()
    assert np.allclose(dsa.rms_norm(q, gamma, eps), ref, rtol=1e-13, atol=1e-13)
    one = dsa.rms_norm(q, np.ones(32), eps)
    ms = np.mean(q * q, axis=-1)
    assert np.allclose(np.mean(one * one, axis=-1), ms / (ms + eps), rtol=1e-13)
