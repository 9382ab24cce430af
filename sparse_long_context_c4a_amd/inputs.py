"""Seeded synthetic inputs for one layer step (decode token or prefill chunk).

This module only draws random numbers and stores them in the storage
formats (f32, bf16 bit patterns, fp8 e4m3fn codes); it contains none of the
layer's arithmetic.  Conversions to bf16 / fp8 use torch's CPU dtype casts.
Both the HIP library's tests and the oracle consume exactly these arrays.

Value recipe (all from ``numpy.random.Generator(PCG64(seed))``, drawn in
the fixed order listed in ``layer_inputs``):

* activations, cached entries, raw tokens, queries, logits, head weights:
  standard normal (float32 draws), stored as f32 or rounded to bf16;
* fp8 tensors (indexer keys, indexer queries): codes = e4m3fn(clip(64 g,
  +-448)) for g standard normal, with one positive f32 scale per row drawn
  as (1 + U[0, 0.25)) / 64, so the dequantised values are about N(0, 1);
* fp4 tensors (MXFP4 indexer keys; their queries are fp8): each E2M1 code
  drawn directly, magnitude code 0..7 with probabilities FP4_MAG_P and a
  fair sign bit, and one E8M0 scale byte per 32 elements uniform in
  {126, 127, 128} (block scales 1/2, 1, 2), so the dequantised values are of
  unit order.  The codes come from no quantisation: a stored MXFP4 cache is
  any codes and scale bytes.

A "random" state stands for a context that was processed earlier: cache
slots j < n_complete(p0) hold random entries, the compressor rings hold the
S raw tokens before p0 and the window ring holds W rotated tokens before
p0 (drawn as random vectors; the layer treats them as opaque stored values).
An "empty" state (p0 = 0) starts a sequence from nothing.

Clustered scores (``Workload.cluster`` > 0, random state with an indexer):
after every other draw, one start per sequence is drawn uniformly from
[0, n_complete(p0) - cluster] and the indexer key scales of the cluster
entries from there are multiplied by 16, so their scores are 16 times
larger and the positive ones crowd the row's Top-k into a few waves.
"""

import numpy as np
import torch

from .configs import Workload

FP8_CODE_GAIN = 64.0
# magnitude codes 0..7 of the drawn fp4 elements (0, 0.5, 1, 1.5, 2, 3, 4, 6)
FP4_MAG_P = np.array([0.10, 0.20, 0.18, 0.15, 0.13, 0.12, 0.08, 0.04])
MX_BLOCK = 32


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def to_bf16_bits(a32):
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_fp8_codes(a32):
    a = np.clip(np.asarray(a32, np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def draw(rng, shape, dtype):
    """One tensor in a storage dtype: f32 array, bf16 uint16 bits, or fp8
    (codes uint8, per-row f32 scales over the last axis)."""
    if dtype == "f32":
        return _normal(rng, shape)
    if dtype == "bf16":
        return to_bf16_bits(_normal(rng, shape))
    if dtype == "fp8":
        codes = to_fp8_codes(_normal(rng, shape) * FP8_CODE_GAIN)
        scales = ((1.0 + 0.25 * rng.random(shape[:-1], dtype=np.float32))
                  / np.float32(FP8_CODE_GAIN)).astype(np.float32)
        return codes, scales
    if dtype == "fp4":  # (codes uint8 0..15 [..., n], scale bytes [..., n / 32])
        mag = rng.choice(8, size=shape, p=FP4_MAG_P)
        sign = rng.integers(0, 2, size=shape) * 8
        scales = rng.integers(126, 129, size=shape[:-1] + (shape[-1] // MX_BLOCK,))
        return (mag | sign).astype(np.uint8), scales.astype(np.uint8)
    raise ValueError(dtype)


def zeros(shape, dtype):
    if dtype == "f32":
        return np.zeros(shape, np.float32)
    if dtype == "bf16":
        return np.zeros(shape, np.uint16)
    if dtype == "fp8":
        return np.zeros(shape, np.uint8), np.zeros(shape[:-1], np.float32)
    if dtype == "fp4":
        return np.zeros(shape, np.uint8), np.zeros(shape[:-1] + (shape[-1] // MX_BLOCK,), np.uint8)
    raise ValueError(dtype)


def _complete(L, s, S):
    return 0 if L < S else (L - S) // s + 1


def raw_idx_dtype(w: Workload):
    """Raw indexer tokens are bf16 when the indexer cache is fp8 or fp4."""
    return "f32" if w.idx_dtype == "f32" else "bf16"


def q_idx_dtype(w: Workload):
    """Indexer queries: fp8 beside fp4 keys, else the keys' storage."""
    return "fp8" if w.idx_dtype == "fp4" else w.idx_dtype


def layer_inputs(w: Workload, seed=None, p0=None, T=None, state="random",
                 e_cap=None):
    """Inputs of one layer step over raw positions p0 .. p0+T-1 for each of
    the w.B sequences.  Decode defaults: p0 = L-1, T = 1.

    Returns a dict of NumPy arrays (storage bits) and ints.  Per-sequence
    tensors have a leading [B] axis.
    """
    seed = w.seed if seed is None else seed
    if p0 is None:
        p0 = w.L - 1 if w.mode == "decode" else w.p0
    if T is None:
        T = 1 if w.mode == "decode" else w.T
    if state == "empty" and p0 != 0:
        raise ValueError("an empty state starts at position 0")
    rng = _rng(seed)
    B, D, Di, H, Hi, S = w.B, w.D, w.Di, w.H, w.Hi, w.S
    E_cap = e_cap if e_cap is not None else -(-(p0 + T) // w.s)
    j0 = _complete(p0, w.s, S)
    n_new = _complete(p0 + T, w.s, S) - j0
    has_idx = Hi > 0
    rdt = raw_idx_dtype(w)
    out = dict(p0=p0, T=T, E_cap=E_cap, j0=j0, n_new=n_new, seed=seed)

    # 1. main cache, 2. indexer cache (+ scales)
    mcd = w.main_cache_dtype or w.main_dtype
    main_cache = zeros((B, E_cap, D), mcd)
    if state == "random" and j0 > 0:
        for b in range(B):
            v = draw(rng, (j0, D), mcd)
            if mcd == "fp8":
                main_cache[0][b, :j0], main_cache[1][b, :j0] = v
            else:
                main_cache[b, :j0] = v
    if mcd == "fp8":
        out["main_cache"], out["main_scale"] = main_cache
    else:
        out["main_cache"], out["main_scale"] = main_cache, None
    out["idx_mx"] = None
    if has_idx:
        ic = zeros((B, E_cap, Di), w.idx_dtype)
        if state == "random" and j0 > 0:
            for b in range(B):
                v = draw(rng, (j0, Di), w.idx_dtype)
                if w.idx_dtype in ("fp8", "fp4"):
                    ic[0][b, :j0], ic[1][b, :j0] = v
                else:
                    ic[b, :j0] = v
        if w.idx_dtype == "fp8":
            out["idx_cache"], out["idx_scale"] = ic
        elif w.idx_dtype == "fp4":
            (out["idx_cache"], out["idx_mx"]), out["idx_scale"] = ic, None
        else:
            out["idx_cache"], out["idx_scale"] = ic, None
    else:
        out["idx_cache"], out["idx_scale"] = None, None

    # 3. compressor rings, 4. window ring
    if state == "random":
        out["main_ring"] = draw(rng, (B, S, D), w.main_dtype)
        out["idx_ring"] = draw(rng, (B, S, Di), rdt) if has_idx else None
        out["win_ring"] = draw(rng, (B, w.W_cap, D), w.main_dtype)
    else:
        out["main_ring"] = zeros((B, S, D), w.main_dtype)
        out["idx_ring"] = zeros((B, S, Di), rdt) if has_idx else None
        out["win_ring"] = zeros((B, w.W_cap, D), w.main_dtype)

    # 5. chunk raw tokens, 6. compressor logits
    out["x"] = draw(rng, (B, T, D), w.main_dtype)
    out["kx"] = draw(rng, (B, T, Di), rdt) if has_idx else None
    out["logits_main"] = _normal(rng, (B, n_new, S))
    out["logits_idx"] = _normal(rng, (B, n_new, S)) if has_idx else None

    # 7. queries, indexer queries (+ scales), head weights
    out["q"] = draw(rng, (B, T, H, D), w.main_dtype)
    if has_idx:
        qdt = q_idx_dtype(w)
        v = draw(rng, (B, T, Hi, Di), qdt)
        if qdt == "fp8":
            out["qi"], out["qi_scale"] = v
        else:
            out["qi"], out["qi_scale"] = v, None
        out["wt"] = _normal(rng, (B, T, Hi))
    else:
        out["qi"] = out["qi_scale"] = out["wt"] = None

    # 8. clustered high scores
    if w.cluster and has_idx and state == "random" and j0 > w.cluster and out["idx_scale"] is not None:
        out["cluster_start"] = []
        for b in range(B):
            start = int(rng.integers(0, j0 - w.cluster + 1))
            out["idx_scale"][b, start:start + w.cluster] *= np.float32(16.0)
            out["cluster_start"].append(start)
    return out


def random_indices(seed, Bq, k, n_vis, fill=1.0):
    """Distinct random entry indices per row (for testing attention alone):
    about fill*min(k, n_vis) valid indices in random order, -1 padded."""
    rng = _rng(seed)
    idx = np.full((Bq, k), -1, np.int32)
    for b in range(Bq):
        nv = int(n_vis[b])
        cnt = min(k, nv, int(round(fill * min(k, nv))))
        if cnt > 0:
            sel = rng.choice(nv, size=cnt, replace=False).astype(np.int32)
            pos = rng.choice(k, size=cnt, replace=False)
            idx[b, pos] = sel
    return idx
