"""Shared pieces of the GPU parity tests: oracle set-up from a workload and
the comparison rules.

Tolerances (stated by the layer's accuracy targets): attention outputs within
max-abs 2e-2 for bf16 storage and 1e-4 for the f32 workload; Top-k index sets
equal except for entries whose oracle score lies within 1e-5 (relative) of
the oracle's k-th score; counts, visibility and -1 padding bit-exact.
"""

import numpy as np
import torch

from oracle import dsa as odsa
from oracle.layer import Geometry

ATOL = {"f32": 1e-4, "bf16": 2e-2}
# log-sum-exp of the logits.  Both sides hold the rotated query in the
# storage dtype (the pages rotate and quantise the query in one step before
# the attention: "DeepSeek V4 稀疏注意力完全解剖", 全景图 step A), so what is
# left is f32 summation (~1e-6) and the rare query element whose f32 and
# fp64 rotations round to neighbouring bf16 values: one such element moves
# a logit by at most 2^-8 |q_d| |v_d| / sqrt(D) ~ 2e-4 for N(0,1) data.
LSE_ATOL = {"f32": 1e-4, "bf16": 1e-3}
TOPK_REL = 1e-5


def geometry(w, **over):
    d = dict(s=w.s, S=w.S, D=w.D, r=w.r, Di=w.Di, r_idx=w.r_idx, H=w.H, Hi=w.Hi, k=w.k, W=w.W,
             base=w.base, base_idx=w.base, main_dtype=w.main_dtype, idx_dtype=w.idx_dtype,
             main_cache_dtype=w.main_cache_dtype)
    d.update(over)
    return Geometry(**d)


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def check_topk_row(gpu_row, scores, k, label=""):
    """GPU index row (any order, -1 padded) against the oracle's scores of the
    visible entries.  Returns the number of tie-swapped entries."""
    gpu_row = np.asarray(gpu_row)
    n = len(scores)
    want = min(k, n)
    sel = gpu_row[gpu_row >= 0]
    assert len(sel) == want, f"{label}: {len(sel)} selected, expected {want}"
    # the selection fills the first min(k, n_vis) places, then -1 padding
    assert np.all(gpu_row[:want] >= 0), f"{label}: padding inside the selection"
    assert np.all(gpu_row[want:] == -1), f"{label}: padding is not -1"
    assert len(np.unique(sel)) == len(sel), f"{label}: duplicate indices"
    assert np.all(sel < n), f"{label}: index beyond n_vis"
    if want == n:
        return 0
    oidx, _ = odsa.topk(scores, k)
    oset = set(oidx[oidx >= 0].tolist())
    gset = set(sel.tolist())
    diff = oset ^ gset
    if diff:
        kth = np.sort(scores)[::-1][want - 1]
        tol = TOPK_REL * max(abs(kth), 1e-30)
        bad = [j for j in diff if abs(scores[j] - kth) > tol]
        assert not bad, f"{label}: entries {bad[:5]} differ beyond tie tolerance"
    return len(diff) // 2


# Largest error seen per kind over the session: kind -> (err, bound, label).
# The test session prints them at the end (tests/conftest.py).
MAXERR = {}


def note_err(kind, err, bound, label):
    cur = MAXERR.get(kind)
    if cur is None or err > cur[0]:
        MAXERR[kind] = (float(err), float(bound), label)


def check_close(gpu, ref, atol, label="", kind=None):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu) == np.isfinite(ref)), f"{label}: non-finite mismatch"
    fin = np.isfinite(ref)
    err = np.max(np.abs(gpu[fin] - ref[fin])) if fin.any() else 0.0
    if kind:
        note_err(kind, err, atol, label)
    assert err <= atol, f"{label}: max abs err {err:.3e} > {atol:.1e}"
    return err


def check_fp8_heads(codes, scales, ref, err, label=""):
    """fp8 output of one row ([H, D] codes, [H] scales) against the oracle's
    values ref [H, D]: each scale is max|ref_h| / 448 within err / 448 (err =
    the attention's own absolute error before rounding), each decoded value
    within half an e4m3fn grid step (taken at |ref| + err, the larger binade
    the kernel's value can fall in) plus err; an all-zero head gives scale 0
    and zero codes."""
    from oracle import codecs as oc
    from oracle import dsa as odsa
    codes = np.asarray(codes)
    gsc = np.asarray(scales, np.float64)
    ref = np.asarray(ref, np.float64)
    _, osig = odsa.quantize_fp8_heads(ref)
    assert np.all(np.abs(gsc - osig) <= err / 448.0 + 1e-6 * osig), f"{label}: scales"
    deq = oc.fp8_decode(codes) * gsc[:, None]
    gs = np.maximum(gsc[:, None], 1e-300)
    x = np.where(gsc[:, None] > 0, (np.abs(ref) + err) / gs, 0.0)
    step = np.where(x < 2 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(x, 1e-300))) - 3))
    tol = (0.5 + 1e-3) * step * gsc[:, None] + err
    bad = np.abs(deq - ref) - tol
    assert np.all(bad <= 0), f"{label}: fp8 output off by {np.max(bad):.3e} beyond the bound"
    zero = ~np.any(ref, axis=1)
    assert not codes[zero].any() and not gsc[zero].any(), f"{label}: zero heads"
