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
# log-sum-exp of the logits: with bf16 storage the rotated query is rounded to
# bf16 before the matrix-core product (relative error <= 2^-9 per element), so
# a logit tau * q.v of N(0,1) data moves by about tau * |q| |v| 2^-9 / sqrt(3)
# ~ 1e-3 and by at most ~4e-2; 1e-2 is taken.  f32 keeps the f32 bound.
LSE_ATOL = {"f32": 1e-4, "bf16": 1e-2}
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
    assert np.all(gpu_row[want:] == -1) or len(sel) == want, label
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


def check_close(gpu, ref, atol, label=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu) == np.isfinite(ref)), f"{label}: non-finite mismatch"
    fin = np.isfinite(ref)
    err = np.max(np.abs(gpu[fin] - ref[fin])) if fin.any() else 0.0
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
