"""fp64 CPU oracle for the c4a / c128a compressed sparse attention layer.

Test infrastructure only (see the package docstring).  Every function works
on float64 NumPy arrays (inputs decoded from their storage bits by
``oracle.codecs``) and follows the pages' description step by step, with no
blocking, fusion or reordering beyond what that description states.

Sources (cited by page title and section):

* [P1] "DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" (gentlecold.top)
* [P2] "DeepSeek V4 稀疏注意力完全解剖" (zoe.im)

Notation: D latent dim, r rotary dims (the last r of D), s stride, S span
(c4a: s=4, S=8; c128a: s=S=128), W window (128), m query position,
H query heads, Hi / Di indexer heads / dim.

Readings where the pages are silent or garbled (each also listed in the
design notes):

* RoPE acts on interleaved pairs of the last r dims with frequencies
  base^(-2i/r).  The pages only fix the relative-position identity
  R_m R_n^T = R_(m-n); the layout itself is a convention -- parity unpinned
  for the layout, pinned for the identities.
* A compressed entry j is rotated at the position of its first raw token,
  s*j (+ offset) -- parity unpinned (any s*j + const satisfies the
  translation-invariance pin).
* The compression weights are one softmax over S logits per entry, shared
  across D.
* The indexer score is sum_h w_h * ReLU(q_h . k_j); w is per (query, head);
  the window is never scored.
* Top-k ties break toward the lower entry index.
* The window [m-W, m-1] excludes m; one joint softmax runs over the selected
  entries and the window tokens.
* Softmax scale 1/sqrt(D).
* Token-wise fp8 (indexer keys; the optional fp8 main cache of decode; the
  optional fp8 attention output, per query and head): one f32 scale per
  vector, max|v| / 448, e4m3fn codes rounded to nearest even.  The pages
  name the formats but give no scale rule for the main cache or the output.
"""

import numpy as np

from . import codecs

# ---------------------------------------------------------------- O1 RoPE


def rope_theta(r, base):
    """Frequencies theta_i = base^(-2i/r), i < r/2 (original RoPE form; [P2]
    references list the RoPE paper)."""
    i = np.arange(r // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / r)


def rope_rotate(x, pos, r, base):
    """Apply R_pos to the last r dims of x (interleaved pairs).

    x: [..., D] float64; pos: scalar or array broadcastable to x.shape[:-1]
    (may be negative: R_(-p) = R_p^{-1}).  The other D-r dims pass through.
    Pair (a, b) = (x[D-r+2i], x[D-r+2i+1]) maps to
    (a cos(p theta_i) - b sin(p theta_i), a sin(p theta_i) + b cos(p theta_i)).
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    if r == 0:
        return out
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_theta(r, base)
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., D - r::2]
    b = x[..., D - r + 1::2]
    out[..., D - r::2] = a * c - b * s
    out[..., D - r + 1::2] = a * s + b * c
    return out


def rope_inverse(x, pos, r, base):
    """R_pos^{-1} x = R_(-pos) x ([P2] 深潜: 为什么必须做 Inverse RoPE)."""
    return rope_rotate(x, -np.asarray(pos, dtype=np.float64), r, base)


# ---------------------------------------------------- O3 counts, O4 window


def n_complete(L, s, S):
    """Entries whose S raw tokens all lie in [0, L): entry j covers
    t_{s j} .. t_{s j + S - 1} ([P2] 机制二: T0 = t0..t7, T1 = t4..t11 for
    c4a; 128 tokens at stride 128 for c128a).  Floor division, so L < S gives
    0."""
    if L < S:
        return 0
    return (L - S) // s + 1


def n_vis(m, s, S):
    """Entries visible to the query at position m: entry j is visible iff its
    last raw token s j + S - 1 < m (causality, [P2] 机制四: the first c128a
    entry, covering 0..127, is invisible to early queries)."""
    return n_complete(m, s, S)


def n_slots(L, s):
    """Cache slots for L raw tokens: one per stride, ceil(L/s) ([P1] 18.2:
    1,048,576 / 4 = 262,144; [P1] 6.1: 256 raw tokens -> 64 c4a slots)."""
    return -(-L // s)


def window_range(m, W):
    """Raw positions in the sliding window of query m: [max(0, m-W), m-1]
    ([P2] 机制四).  Returned as a half-open Python range."""
    return range(max(0, m - W), m)


# ------------------------------------------------------------ O2 compress


def softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def compress_entry(tokens, logits, pos, r, base, gamma=None, eps=1e-6):
    """One compressed entry ([P1] 5.2; [P2] 机制二).

    tokens: [S, D] raw tokens t_{s j} .. t_{s j + S - 1}; logits: [S].
    The entry is the softmax-weighted sum of its S raw tokens, optionally
    RMS-normalised (the pages' fused order is compress -> RMSNorm -> RoPE ->
    insert, [P2] 融合点 1), then rotated at ``pos``.
    """
    w = softmax(logits)
    c = w @ np.asarray(tokens, dtype=np.float64)
    if gamma is not None:
        c = np.asarray(gamma, dtype=np.float64) * c / np.sqrt(np.mean(c * c) + eps)
    return rope_rotate(c, pos, r, base)


def rms_norm(x, gamma, eps):
    """RMSNorm over the last axis: gamma * x / sqrt(mean(x^2) + eps).  The
    pages name a Q-norm ahead of the attention ([P2] 融合点 3: "Q Norm", fused
    with the window keys' RoPE and insert) without its formula; the reading
    taken is the same RMSNorm the compressor uses ([P2] 融合点 1)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, np.float64) * x / np.sqrt(ms + eps)


def quantize_fp8_entry(c):
    """Token-wise fp8 ([P2] 第三层: decode uses token-wise fp8): one fp32
    scale per entry, sigma = max|c| / 448, codes = RNE_e4m3fn(c / sigma).
    The scale is rounded to fp32 first, as it is stored in fp32; an all-zero
    entry gets sigma = 0 and zero codes.  Returns (codes uint8, sigma f64)."""
    c = np.asarray(c, dtype=np.float64)
    amax = np.max(np.abs(c))
    sigma = float(np.float32(amax / codecs.FP8_MAX))
    if sigma == 0.0:
        return np.zeros(c.shape, dtype=np.uint8), 0.0
    return codecs.fp8_encode(c / sigma), sigma


MX_BLOCK = 32  # elements sharing one E8M0 scale (OCP MX)


def quantize_mxfp4(c):
    """MXFP4 ([P2] 第三层 "indexer 用 fp4"; [P2] 机制三: the indexer is light
    because it is stored in fp4).  The pages name the precision only; the
    reading taken is the OCP Microscaling (MX) FP4 format: blocks of 32
    consecutive elements share an E8M0 scale X = 2^e, with the spec's
    conversion e = floor(log2(max|block|)) - 2 (2 = the largest E2M1
    exponent), clamped to [-127, 127], e = -127 for an all-zero block; each
    element is the E2M1 code of v / X (nearest, ties to even, saturating at
    6).  c: [..., D] with D a multiple of 32.  Returns (codes uint8 [..., D],
    scale bytes uint8 [..., D / 32] = e + 127)."""
    c = np.asarray(c, dtype=np.float64)
    blk = c.reshape(c.shape[:-1] + (c.shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))  # amax = f 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, np.clip(ex - 1 - 2, -127, 127), -127)
    codes = codecs.fp4_encode(blk / np.ldexp(1.0, e)[..., None])
    return codes.reshape(c.shape), (e + 127).astype(np.uint8)


def mxfp4_decode(codes, scales):
    """MXFP4 codes [..., D] and scale bytes [..., D / 32] -> float64."""
    v = codecs.fp4_decode(codes)
    blk = v.reshape(v.shape[:-1] + (v.shape[-1] // MX_BLOCK, MX_BLOCK))
    x = np.ldexp(1.0, np.asarray(scales).astype(np.int64) - 127)
    return (blk * x[..., None]).reshape(v.shape)


def compress_range(token_at, logits, j0, n, s, S, r, base, pos_offset=0,
                   gamma=None, eps=1e-6):
    """Entries j0 .. j0+n-1.  ``token_at(p)`` returns raw token p (float64
    [D]); logits: [n, S].  Entry j is rotated at s*j + pos_offset.
    Returns [n, D] float64 (before any storage rounding)."""
    out = []
    for e in range(n):
        j = j0 + e
        toks = np.stack([token_at(s * j + i) for i in range(S)])
        out.append(compress_entry(toks, logits[e], s * j + pos_offset, r, base,
                                  gamma, eps))
    if not out:
        return np.zeros((0, 0))
    return np.stack(out)


# ------------------------------------------------------------- O5 indexer


def indexer_scores(q, w, keys):
    """Lightning-indexer scores ([P1] 4.1; score form sum_h w_h ReLU(q_h.k_s)).

    q: [Hi, Di], w: [Hi], keys: [n, Di] (dequantised, float64).
    Returns I: [n] with I_j = sum_h w_h * max(0, q_h . k_j).
    """
    dots = np.asarray(keys, np.float64) @ np.asarray(q, np.float64).T  # [n, Hi]
    return np.maximum(dots, 0.0) @ np.asarray(w, np.float64)


# --------------------------------------------------------------- O6 top-k


def topk(scores, k):
    """S_t = TopK(I_{t,:}, k) ([P1] 4.2).

    Visible entries are ordered by score descending, ties by lower index;
    the first min(k, n) are kept.  Returned as ascending indices padded with
    -1 to length k, plus the kept scores in the same order (NaN padded)."""
    scores = np.asarray(scores, np.float64)
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))  # primary: -score, then index
    keep = np.sort(order[:min(k, n)])
    idx = np.full(k, -1, dtype=np.int64)
    idx[:keep.size] = keep
    sc = np.full(k, np.nan)
    sc[:keep.size] = scores[keep]
    return idx, sc


# ----------------------------------------------------------- O7 attention


def sparse_attention(q_rot, vecs, m_pos, r, base, scale):
    """MQA attention over the gathered set with K = V and inverse RoPE.

    q_rot: [H, D] query already rotated at m; vecs: [A, D] the gathered
    vectors (selected compressed entries and window tokens, each carrying its
    own rotation), shared by all H heads ([P1] 4.3 MQA mode; [P1] 5.1 and
    [P2] 机制一 K/V sharing).  One joint softmax over the whole set.
    Output o_h = sum_a p_a v_a, then out_h = R_m^{-1} o_h ([P2] 深潜 Inverse
    RoPE).  Returns (out [H, D], lse [H]) with lse the natural-log sum of
    exp(logits); an empty set gives zeros and -inf.
    """
    q_rot = np.asarray(q_rot, np.float64)
    H, D = q_rot.shape
    if vecs is None or len(vecs) == 0:
        return np.zeros((H, D)), np.full(H, -np.inf)
    vecs = np.asarray(vecs, np.float64)
    logits = scale * (q_rot @ vecs.T)  # [H, A]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    z = e.sum(axis=1, keepdims=True)
    o = (e / z) @ vecs
    lse = (mx + np.log(z))[:, 0]
    return rope_inverse(o, m_pos, r, base), lse


def quantize_fp8_heads(out):
    """fp8 attention output ([P2] 融合点 2: the inverse RoPE and the fp8
    quantisation that feeds the o_lora projection fused in one pass).  The
    pages give no scale rule for this tensor; the reading taken is the decode
    KV's token-wise one ([P2] 第三层), one scale per (query, head) vector:
    each row of ``out`` [H, D] goes through ``quantize_fp8_entry``.
    Returns (codes uint8 [H, D], sigma float64 [H])."""
    out = np.asarray(out, np.float64)
    q = [quantize_fp8_entry(v) for v in out]
    return np.stack([c for c, _ in q]), np.array([sg for _, sg in q], np.float64)


def gather_set(m, idx, entries, window_vec, W):
    """The attention set A(m): the selected compressed entries (idx >= 0) and
    the window tokens n in [m-W, m-1] ([P2] 机制四; [P1] flowchart: Top-k
    entries and the SWA KV both feed one Main Attention).
    ``window_vec(n)`` returns the stored rotated vector of raw token n."""
    sel = [entries[j] for j in idx if j >= 0]
    win = [window_vec(n) for n in window_range(m, W)]
    if not sel and not win:
        return None  # empty set
    return np.array(sel + win, dtype=np.float64)
