"""fp64 oracle of one layer step (decode token or prefill chunk).

Test infrastructure only (see the package docstring).

Per-layer dataflow as the pages draw it ([P1] "DeepSeek DSA、DeepSeek V4与
vLLM Hybrid KV Cache详解", 15 flowchart; [P2] "DeepSeek V4 稀疏注意力完全解剖",
全景图 step C-E): the compressor turns raw tokens into compressed entries
(main KV and the indexer's own keys), the lightning indexer scores every
visible entry, Top-k keeps k of them, and one main attention runs over the
kept entries plus the raw sliding window, with the inverse rotation on the
output.

State kept between steps ([P1] 6 / [P2] 设计 2): the main and indexer
caches (slot j holds entry j), the compressor state = the last S raw tokens
(c4a 8, c128a 128) for each compressor, and the window of rotated raw tokens.

A decode step is a chunk of one token: the entry completing at m (if any) is
compressed first, then the query at m runs.  Entries completing inside a
chunk are visible to the chunk's later queries; the window excludes m, so
the token at m is inserted after its own attention.

Storage rounding is applied exactly where the method stores a value: new
cache entries (f32 / bf16 / token-wise fp8) and inserted window tokens.
"""

from dataclasses import dataclass, field

import numpy as np

from . import codecs
from . import dsa


def store(v, dtype):
    """Round a float64 vector (or rows) to what a cache of ``dtype`` holds and
    return the decoded float64 value (plus the fp8 scale, else None)."""
    v = np.asarray(v, np.float64)
    if dtype == "f64":  # no rounding (used to state exact invariances)
        return v.copy(), None
    if dtype == "f32":
        return v.astype(np.float32).astype(np.float64), None
    if dtype == "bf16":
        return codecs.bf16_decode(codecs.bf16_encode(v)), None
    if dtype == "fp8":
        codes, sigma = dsa.quantize_fp8_entry(v)
        return sigma * codecs.fp8_decode(codes), sigma
    if dtype == "fp4":  # MXFP4: the block scales are part of the value
        codes, sc = dsa.quantize_mxfp4(v)
        return dsa.mxfp4_decode(codes, sc), None
    raise ValueError(dtype)


@dataclass
class Geometry:
    s: int
    S: int
    D: int
    r: int
    Di: int
    r_idx: int
    H: int
    Hi: int
    k: int
    W: int
    base: float = 10000.0
    base_idx: float = 10000.0
    pos_offset: int = 0
    main_dtype: str = "bf16"   # main cache and window
    main_cache_dtype: str = ""  # "fp8": token-wise fp8 main cache; "": main_dtype
    idx_dtype: str = "fp8"     # indexer cache
    scale: float = None        # softmax scale; None -> 1/sqrt(D)
    gamma: np.ndarray = None   # optional RMSNorm weight of the main compressor
    gamma_idx: np.ndarray = None
    q_gamma: np.ndarray = None  # optional Q-norm weight (each query head, before rotation)
    eps: float = 1e-6

    @property
    def tau(self):
        return self.scale if self.scale is not None else 1.0 / np.sqrt(self.D)


@dataclass
class SeqState:
    """One sequence's layer state, all values decoded to float64."""
    main_cache: np.ndarray      # [E_cap, D]
    idx_cache: np.ndarray       # [E_cap, Di]
    idx_scale: np.ndarray       # [E_cap] (fp8 scales; ones otherwise)
    main_ring: np.ndarray       # [S, D]   raw token p at slot p mod S
    idx_ring: np.ndarray        # [S, Di]
    win_ring: np.ndarray        # [W_cap, D] rotated token n at slot n mod W_cap
    entries_written: list = field(default_factory=list)
    alt_out: dict = field(default_factory=dict)


def layer_chunk(g: Geometry, st: SeqState, p0, X, KX, logits_main, logits_idx,
                Q, QI, WT, rotate_q=True, only=None, alt_idx=None):
    """Run the layer over raw tokens p0 .. p0+T-1 of one sequence.

    X [T, D], KX [T, Di] raw (un-rotated) tokens for the main and indexer
    compressors; logits_main / logits_idx [n_new, S] for the entries that
    complete in the chunk, j = n_complete(p0) .. n_complete(p0+T)-1;
    Q [T, H, D] queries (rotated here at their position when rotate_q);
    QI [T, Hi, Di] dequantised indexer queries; WT [T, Hi] head weights.
    Tokens before p0 come from the compressor rings (which must hold
    positions p0-S .. p0-1) and the window ring.

    A layer without an indexer (Hi = 0, the c128a case) selects every
    visible entry, which needs k >= n_vis ([P2] 机制三: c128a k = 8192 over
    8K entries is full attention).  ``only``: optional iterable of chunk
    offsets whose outputs are computed (the state update is always full).

    The rotated query R_m q is held in the layer's storage dtype before the
    logits: the pages rotate and quantise the query in one fused step ahead
    of the attention ([P2] 全景图, decode step A: "Q RoPE + quant").  With
    ``g.q_gamma`` each head is RMS-normalised first ([P2] 融合点 3, "Q Norm").

    ``alt_idx`` [T, k] (optional): another selection per row, already checked
    against this one under the tie rule; where its set differs, the
    attention is also evaluated on it (stepwise parity: the attention of a
    row whose Top-k took an allowed tie swap is compared on the set actually
    chosen).  Those results go to ``st.alt_out`` as {t: (out, lse)}.

    Returns (out [T, H, D], lse [T, H], idx [T, k]) and updates ``st`` in
    place.
    """
    X = np.asarray(X, np.float64)
    KX = np.asarray(KX, np.float64)
    T = X.shape[0]
    s, S, W = g.s, g.S, g.W
    off = g.pos_offset
    W_cap = st.win_ring.shape[0]

    def tok_main(p):
        return X[p - p0] if p >= p0 else st.main_ring[p % S]

    def tok_idx(p):
        return KX[p - p0] if p >= p0 else st.idx_ring[p % S]

    # S1: compress every entry that completes inside the chunk.
    j0 = dsa.n_complete(p0, s, S)
    j1 = dsa.n_complete(p0 + T, s, S)
    n_new = j1 - j0
    if n_new:
        main_new = dsa.compress_range(tok_main, logits_main, j0, n_new, s, S, g.r,
                                      g.base, off, g.gamma, g.eps)
        idx_new = None
        if g.Hi > 0:
            idx_new = dsa.compress_range(tok_idx, logits_idx, j0, n_new, s, S, g.r_idx,
                                         g.base_idx, off, g.gamma_idx, g.eps)
        for e in range(n_new):
            j = j0 + e
            st.main_cache[j], _ = store(main_new[e], g.main_cache_dtype or g.main_dtype)
            if idx_new is not None:
                val, sig = store(idx_new[e], g.idx_dtype)
                st.idx_cache[j] = val
                st.idx_scale[j] = 1.0 if sig is None else sig
        st.entries_written.append((j0, n_new, main_new, idx_new))

    # Rotated window tokens of this chunk, as the window stores them.
    chunk_win = {}

    def win_vec(n):
        if n >= p0:
            if n not in chunk_win:
                chunk_win[n], _ = store(dsa.rope_rotate(X[n - p0], n + off, g.r, g.base),
                                        g.main_dtype)
            return chunk_win[n]
        return st.win_ring[n % W_cap]

    outs = np.zeros((T, g.H, g.D))
    lses = np.zeros((T, g.H))
    idxs = np.full((T, g.k), -1, dtype=np.int64)
    todo = range(T) if only is None else sorted(set(only))
    for t in todo:
        m = p0 + t
        nv = dsa.n_vis(m, s, S)
        # S3 + S4: indexer over the visible entries, then Top-k.
        if g.Hi > 0:
            scores = dsa.indexer_scores(QI[t], WT[t], st.idx_cache[:nv])
            idx, _ = dsa.topk(scores, g.k)
        else:
            if nv > g.k:
                raise ValueError("a layer without an indexer needs k >= n_vis")
            idx = np.full(g.k, -1, dtype=np.int64)
            idx[:nv] = np.arange(nv)
        idxs[t] = idx
        # S5: attention over the selected entries and the window.
        vecs = dsa.gather_set(m, idx, st.main_cache, win_vec, W)
        if rotate_q:
            qt = Q[t] if g.q_gamma is None else dsa.rms_norm(Q[t], g.q_gamma, g.eps)
            q, _ = store(dsa.rope_rotate(qt, m + off, g.r, g.base), g.main_dtype)
        else:
            q = np.asarray(Q[t], np.float64)
        outs[t], lses[t] = dsa.sparse_attention(q, vecs, m + off, g.r, g.base, g.tau)
        if alt_idx is not None:
            alt = np.asarray(alt_idx[t])
            if set(alt[alt >= 0].tolist()) != set(idx[idx >= 0].tolist()):
                avecs = dsa.gather_set(m, alt, st.main_cache, win_vec, W)
                st.alt_out[t] = dsa.sparse_attention(q, avecs, m + off, g.r, g.base, g.tau)

    # State update: compressor rings and window ring take the chunk's tokens.
    for p in range(max(p0, p0 + T - S), p0 + T):
        st.main_ring[p % S] = X[p - p0]
        st.idx_ring[p % S] = KX[p - p0]
    for n in range(max(p0, p0 + T - W_cap), p0 + T):
        st.win_ring[n % W_cap] = win_vec(n)
    return outs, lses, idxs
