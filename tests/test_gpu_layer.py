"""GPU parity of the whole layer step (dsa_layer_decode / dsa_layer_prefill)
against the fp64 oracle run end to end from the same seeded inputs.

Small cases cover edge conditions (a fresh sequence, ragged chunks, a chunk
split into decode steps, c128a without an indexer); the full-size cases are
the five workloads (decode at 64K and 1M, c128a at 1M, the 4096-token
prefill chunk), checked on every row (decode) or on sampled rows
(prefill), in the same launch configuration the benchmark times."""

import numpy as np
import pytest
import torch

from oracle import dsa as odsa
from oracle.run import decode_store, q_dtype_idx, run_layer
from sparse_long_context_c4a_amd import configs, inputs as gen

from gpu_helpers import (ATOL, LSE_ATOL, check_close, check_fp8_heads, check_topk_row,
                         geometry, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layer():
    from sparse_long_context_c4a_amd import layer as Ly
    return Ly


def _compare(w, inp, ores, out, lse, idx, rows=None, label=""):
    """GPU outputs [B, T, ...] against the oracle result dict.  A row whose
    selection differs from the oracle's by allowed ties is compared with the
    oracle's attention over the GPU's set (``_oracle`` with ``alt_idx``)."""
    out, lse, idx = to_np(out), lse.cpu().numpy(), idx.cpu().numpy()
    B, T = out.shape[:2]
    rows = range(T) if rows is None else rows
    st = ores["states"]
    dt = w.main_dtype
    swaps = 0
    for b in range(B):
        keys = None
        if w.Hi > 0 and T > 1:  # decode the chunk's indexer cache once
            keys = st[b].idx_cache[:odsa.n_vis(inp["p0"] + max(rows), w.s, w.S)]
        for t in rows:
            m = inp["p0"] + t
            nv = odsa.n_vis(m, w.s, w.S)
            lab = f"{label} b={b} t={t} m={m}"
            if w.Hi > 0:
                qi = ores["qi_dec"][b][t]
                kv = keys[:nv] if keys is not None else st[b].idx_cache[:nv]
                scores = odsa.indexer_scores(qi, np.asarray(inp["wt"][b][t], np.float64), kv)
                swaps += check_topk_row(idx[b, t], scores, w.k, lab)
                same = set(idx[b, t][idx[b, t] >= 0].tolist()) == \
                    set(ores["idx"][b, t][ores["idx"][b, t] >= 0].tolist())
            else:
                assert sorted(idx[b, t][idx[b, t] >= 0].tolist()) == list(range(nv)), lab
                same = True
            if same:
                ro, rl = ores["out"][b, t], ores["lse"][b, t]
            else:  # the oracle's attention over the set the GPU chose
                ro, rl = st[b].alt_out[t]
                lab += " (GPU set)"
            check_close(out[b, t], ro, ATOL[dt], lab, kind=f"layer out {dt}")
            check_close(lse[b, t], rl, LSE_ATOL[dt], lab + " lse", kind=f"layer lse {dt}")
    return swaps


def _oracle(w, inp, only=None, gpu_idx=None, **geo):
    g = geometry(w, **geo)
    alt = None if gpu_idx is None else np.asarray(gpu_idx.cpu().numpy(), np.int64)
    res = run_layer(g, inp, only=only, alt_idx=alt)
    if w.Hi > 0:
        res["qi_dec"] = [decode_store(inp["qi"][b], q_dtype_idx(w.idx_dtype),
                                      None if inp["qi_scale"] is None else inp["qi_scale"][b])
                         for b in range(inp["x"].shape[0])]
    return res


def _run_gpu(w, inp, decode=None, state=None, **kw):
    Ly = _layer()
    st = state or Ly.state_from_inputs(inp, DEV)
    ch = Ly.chunk_from_inputs(w, inp, DEV)
    out, lse, idx, status, _ = Ly.run(w, st, ch, decode=decode, max_pos_end=st.e_cap * w.s, **kw)
    torch.cuda.synchronize()
    assert status.item() == 0, f"device status {status.item()}"
    return st, out, lse, idx


SMALL = [
    # name, workload, overrides, p0, T, state
    ("c4a_decode_B3_L3000", configs.C4A_DECODE_64K, dict(B=3, L=3000), None, None, "random"),
    ("c4a_decode_L20_tiny", configs.C4A_DECODE_64K, dict(B=2, L=20), None, None, "random"),
    ("c4a_decode_ring_eq_window", configs.C4A_DECODE_64K, dict(B=2, L=2000, w_cap=128), None,
     None, "random"),
    ("c128a_decode_B2_L5000", configs.C128A_DECODE_1M, dict(B=2, L=5000, k=64), None, None,
     "random"),
    ("c4a_prefill_ragged_T77", configs.C4A_PREFILL_128K, dict(L=2077), 2000, 77, "random"),
    ("c4a_prefill_fresh_T300", configs.C4A_PREFILL_128K, dict(L=300), 0, 300, "empty"),
    ("f32_prefill_fresh_T200", configs.TINY_C4A_F32, dict(L=200, mode="prefill"), 0, 200,
     "empty"),
    # MXFP4 indexer cache: a decode step completing an entry (stand-alone
    # prologue), the same with the prologue in the indexer's launch, and a
    # ragged prefill chunk
    ("c4a_decode_fp4_B3_L3000", configs.C4A_DECODE_1M_FP4, dict(B=3, L=3000), None, None,
     "random"),
    ("c4a_decode_fp4_B2_L40000_fused", configs.C4A_DECODE_1M_FP4, dict(B=2, L=40000), None,
     None, "random"),
    ("c4a_prefill_fp4_ragged_T77", configs.C4A_PREFILL_128K, dict(L=2077, idx_dtype="fp4"),
     2000, 77, "random"),
]


@pytest.mark.parametrize("name", ["c4a_decode_B3_L3000", "c128a_decode_B2_L5000",
                                  "c4a_prefill_ragged_T77"])
def test_layer_fp8_out(name):
    """The layer with its output stored as fp8 (fused with the inverse
    rotation): decoded against the oracle's output, rows with the oracle's
    selection."""
    case = next(c for c in SMALL if c[0] == name)
    _, w0, over, p0, T, state = case
    w = configs.shrink(w0, **over)
    seed = 5000 + SMALL.index(case)
    print(f"[dsa_layer fp8 out] {name} B={w.B} p0={p0} T={T} seed={seed}", flush=True)
    inp = gen.layer_inputs(w, seed=seed, p0=p0, T=T, state=state)
    _check_fp8_layer(w, inp, name)


def _check_fp8_layer(w, inp, name):
    Ly = _layer()
    st = Ly.state_from_inputs(inp, DEV)
    ch = Ly.chunk_from_inputs(w, inp, DEV)
    (codes, osc), lse, idx, status, _ = Ly.run(w, st, ch, out_fp8=True,
                                               max_pos_end=st.e_cap * w.s)
    torch.cuda.synchronize()
    assert status.item() == 0, f"device status {status.item()}"
    ores = _oracle(w, inp, gpu_idx=idx)
    codes, osc, idx = codes.cpu().numpy(), osc.cpu().numpy(), idx.cpu().numpy()
    for b in range(w.B):
        for t in range(codes.shape[1]):
            if w.Hi > 0:  # the GPU's set passes the tie rule first
                nv = odsa.n_vis(inp["p0"] + t, w.s, w.S)
                scores = odsa.indexer_scores(ores["qi_dec"][b][t],
                                             np.asarray(inp["wt"][b][t], np.float64),
                                             ores["states"][b].idx_cache[:nv])
                check_topk_row(idx[b, t], scores, w.k, f"{name} b={b} t={t}")
            sel = set(idx[b, t][idx[b, t] >= 0].tolist())
            if sel == set(ores["idx"][b, t][ores["idx"][b, t] >= 0].tolist()):
                ref = ores["out"][b, t]
            else:  # an allowed tie swap: the oracle over the GPU's set
                ref = ores["states"][b].alt_out[t][0]
            check_fp8_heads(codes[b, t], osc[b, t], ref, ATOL[w.main_dtype],
                            f"{name} b={b} t={t}")


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_layer_small(case):
    name, w0, over, p0, T, state = case
    w = configs.shrink(w0, **over)
    seed = 5000 + SMALL.index(case)
    print(f"[dsa_layer] {name} B={w.B} p0={p0} T={T} seed={seed}", flush=True)
    inp = gen.layer_inputs(w, seed=seed, p0=p0, T=T, state=state)
    st, out, lse, idx = _run_gpu(w, inp)
    ores = _oracle(w, inp, gpu_idx=idx)
    _compare(w, inp, ores, out, lse, idx, label=name)
    # the state the layer leaves behind: window ring and compressor rings
    for b in range(w.B):
        ring = to_np(st.main_ring[b])
        check_close(ring, ores["states"][b].main_ring, 0.0, f"{name} main ring")
        win = to_np(st.window[b])
        check_close(win, ores["states"][b].win_ring, ATOL[w.main_dtype] / 4, f"{name} window")
    if w.idx_dtype == "fp4":
        assert _check_fp4_entries(w, st, ores, name) == inp["n_new"] * w.B


def _check_fp4_entries(w, st, ores, name):
    """The indexer entries a step wrote in MXFP4 (codes in the tile layout
    and E8M0 block scales) against the oracle's quantisation of its f64
    entries: scale bytes equal unless a block maximum lies within f32
    rounding of a power of two, each element within its rounding step, and
    the codes equal but for rounding-boundary cases.  Returns the count."""
    Ly = _layer()
    codes = Ly.idx4_rows(st.idx_cache, st.idx_cache.shape[1]).cpu().numpy()
    mx = st.idx_mx.cpu().numpy()
    n = same = tot = 0
    for b in range(w.B):
        for j0, n_new, _, idx_new in ores["states"][b].entries_written:
            for e in range(n_new):
                j, ref = j0 + e, idx_new[e]
                oc, osc = odsa.quantize_mxfp4(ref)
                amax = np.abs(ref).reshape(-1, 32).max(axis=-1)
                lg = np.log2(np.maximum(amax, 1e-300))
                near = np.abs(lg - np.round(lg)) < 1e-5
                assert np.all((mx[b, j] == osc) | near), f"{name} b={b} entry {j} scales"
                x = 2.0 ** (np.repeat(mx[b, j].astype(np.float64), 32) - 127.0)
                am = np.abs(ref) / x
                bound = np.where(am < 2, 0.25, np.where(am < 4, 0.5,
                                                        np.where(am < 6, 1.0, am - 6.0)))
                err = np.abs(odsa.mxfp4_decode(codes[b, j], mx[b, j]) - ref)
                assert np.all(err <= (bound * (1 + 1e-5) + 1e-6) * x), f"{name} b={b} entry {j}"
                same += int(np.sum(codes[b, j] == oc))
                tot += oc.size
                n += 1
    assert tot == 0 or same >= 0.99 * tot, (same, tot)
    return n


def test_tiny_f32_workload_prefill_then_decode():
    """The tiny fp32 workload: a fresh sequence of 1023 raw tokens processed
    as one prefill chunk, then the decode step at position 1023 (k = 64 of
    254 visible entries)."""
    w = configs.TINY_C4A_F32
    print("[dsa_layer] tiny f32: prefill 0..1022 then decode 1023", flush=True)
    wp = configs.shrink(w, mode="prefill")
    inp = gen.layer_inputs(wp, seed=w.seed, p0=0, T=1024, state="empty")
    # split the same token stream into a 1023-token chunk and a 1-token step
    pre = {k: v for k, v in inp.items()}
    dec = {k: v for k, v in inp.items()}
    n_pre = odsa.n_complete(1023, 4, 8)
    for key in ("x", "kx", "q", "qi", "wt"):
        pre[key] = inp[key][:, :1023]
        dec[key] = inp[key][:, 1023:]
    pre["qi_scale"] = dec["qi_scale"] = None
    for key in ("logits_main", "logits_idx"):
        pre[key] = inp[key][:, :n_pre]
        dec[key] = inp[key][:, n_pre:]
    pre.update(T=1023, n_new=n_pre)
    dec.update(p0=1023, T=1, j0=n_pre, n_new=inp["n_new"] - n_pre)
    Ly = _layer()
    st = Ly.state_from_inputs(inp, DEV)
    _, out_p, lse_p, idx_p = _run_gpu(wp, pre, state=st)
    _, out_d, lse_d, idx_d = _run_gpu(w, dec, state=st)
    # oracle: the same two steps on one state
    g = geometry(w)
    from oracle.run import run_layer as rl
    ores_all = rl(g, inp, only=[1022, 1023])
    check_close(to_np(out_d)[0, 0], ores_all["out"][0, 1023], ATOL["f32"], "decode 1023")
    check_close(to_np(out_p)[0, 1022], ores_all["out"][0, 1022], ATOL["f32"], "prefill 1022")
    assert set(idx_d.cpu().numpy()[0, 0].tolist()) == set(ores_all["idx"][0, 1023].tolist())
    assert odsa.n_vis(1023, 4, 8) == 254


def test_chunked_prefill_matches_single_pass():
    """Chunk invariance on the GPU: one 64-token chunk vs chunks of 5, 1, 1,
    13 and 44 tokens (sizes not divisible by the stride) on the same state;
    both against the oracle."""
    w = configs.shrink(configs.C4A_PREFILL_128K, L=3064)
    inp = gen.layer_inputs(w, seed=5100, p0=3000, T=64, state="random")
    print("[dsa_layer] chunked prefill 3000..3063", flush=True)
    Ly = _layer()
    _, out1, lse1, idx1 = _run_gpu(w, inp)
    st = Ly.state_from_inputs(inp, DEV)
    outs = []
    p = 0
    j0 = inp["j0"]
    for T in (5, 1, 1, 13, 44):
        sub = dict(inp)
        a, b = odsa.n_complete(3000 + p, 4, 8), odsa.n_complete(3000 + p + T, 4, 8)
        for key in ("x", "kx", "q", "qi", "qi_scale", "wt"):
            sub[key] = inp[key][:, p:p + T]
        for key in ("logits_main", "logits_idx"):
            sub[key] = inp[key][:, a - j0:b - j0]
        sub.update(p0=3000 + p, T=T, j0=a, n_new=b - a)
        _, o, _, _ = _run_gpu(w, sub, state=st, decode=(T == 1) or None)
        outs.append(to_np(o))
        p += T
    got = np.concatenate(outs, axis=1)
    check_close(got, to_np(out1), 2 * ATOL["bf16"], "chunked vs single")


FULL = [configs.C4A_DECODE_64K, configs.C4A_DECODE_1M, configs.C128A_DECODE_1M,
        configs.C4A_DECODE_1M_CLUSTERED, configs.C4A_DECODE_1M_FP4]


@pytest.mark.parametrize("w", FULL, ids=[w.name for w in FULL])
def test_layer_full_size_decode(w):
    print(f"[dsa_layer_decode] {w.name} full size, seed={w.seed}", flush=True)
    inp = gen.layer_inputs(w)
    st, out, lse, idx = _run_gpu(w, inp)
    ores = _oracle(w, inp, gpu_idx=idx)
    swaps = _compare(w, inp, ores, out, lse, idx, label=w.name)
    assert swaps <= 2
    if w.idx_dtype == "fp4":
        assert _check_fp4_entries(w, st, ores, w.name) == w.B
    if w.cluster:  # a large share of the Top-k sits in a few waves of the cluster
        ix = idx.cpu().numpy()
        for b, c0 in enumerate(inp["cluster_start"]):
            assert np.sum((ix[b, 0] >= c0) & (ix[b, 0] < c0 + w.cluster)) > 100, b


def test_layer_full_size_decode_fp8_out():
    """The 1M-context c4a decode step (B = 4) with its output stored as fp8,
    as the benchmark also times it."""
    w = configs.C4A_DECODE_1M
    print(f"[dsa_layer_decode fp8 out] {w.name} full size, seed={w.seed}", flush=True)
    _check_fp8_layer(w, gen.layer_inputs(w), w.name + " fp8")


def test_layer_full_size_prefill_sampled_rows():
    w = configs.C4A_PREFILL_128K
    print(f"[dsa_layer_prefill] {w.name} full size, seed={w.seed}", flush=True)
    inp = gen.layer_inputs(w)
    _, out, lse, idx = _run_gpu(w, inp)
    # 256 rows spread over the chunk, with both ends
    rows = sorted(set(np.linspace(0, w.T - 1, 248).astype(int).tolist()) |
                  {0, 1, 2, 3, 4, 5, 127, 128, 4092, 4093, 4094, 4095})
    assert len(rows) >= 256
    ores = _oracle(w, inp, only=rows, gpu_idx=idx)
    _compare(w, inp, ores, out, lse, idx, rows=rows, label=w.name)


WRITTEN = [
    # name, workload, overrides, RMSNorm on the compressor
    ("c4a_L3000", configs.C4A_DECODE_64K, dict(B=3, L=3000), False),
    ("c4a_L3000_rmsnorm", configs.C4A_DECODE_64K, dict(B=3, L=3000), True),
    ("c128a_L5120", configs.C128A_DECODE_1M, dict(B=2, L=5120, k=64), False),
    ("c128a_L5120_rmsnorm", configs.C128A_DECODE_1M, dict(B=2, L=5120, k=64), True),
]


@pytest.mark.parametrize("case", WRITTEN, ids=[c[0] for c in WRITTEN])
def test_layer_decode_written_entry(case):
    """The main entry a decode step completes (m + 1 a multiple of s, past
    the first span), as stored in the cache: the decode prologue's compressor
    (split by dims over several workgroups, or whole when the RMSNorm needs
    the full vector) against the oracle's entry before storage rounding."""
    name, w0, over, use_gamma = case
    w = configs.shrink(w0, **over)
    seed = 5600 + WRITTEN.index(case)
    print(f"[dsa_layer written entry] {name} B={w.B} L={w.L} seed={seed}", flush=True)
    inp = gen.layer_inputs(w, seed=seed, state="random")
    rng = np.random.default_rng(seed)
    gam = (1.0 + 0.5 * rng.standard_normal(w.D)).astype(np.float32) if use_gamma else None
    gam_i = (1.0 + 0.5 * rng.standard_normal(w.Di)).astype(np.float32) \
        if use_gamma and w.Hi else None
    Ly = _layer()
    st = Ly.state_from_inputs(inp, DEV)
    ch = Ly.chunk_from_inputs(w, inp, DEV)
    tg = torch.tensor(gam, device=DEV) if gam is not None else None
    tgi = torch.tensor(gam_i, device=DEV) if gam_i is not None else None
    _, _, _, status, _ = Ly.run(w, st, ch, max_pos_end=st.e_cap * w.s, rms_gamma=tg,
                                rms_gamma_idx=tgi)
    torch.cuda.synchronize()
    assert status.item() == 0, f"device status {status.item()}"
    g = geometry(w, gamma=None if gam is None else gam.astype(np.float64),
                 gamma_idx=None if gam_i is None else gam_i.astype(np.float64))
    res = run_layer(g, inp)
    cache = to_np(st.main_cache)
    n = 0
    for b in range(w.B):
        for j0, n_new, main_new, _ in res["states"][b].entries_written:
            for e in range(n_new):
                ref = main_new[e]
                tol = np.abs(ref) * 2.0 ** -8 + 1e-5  # bf16 storage + f32 sums
                err = np.abs(cache[b, j0 + e] - ref) - tol
                assert np.all(err <= 0), f"{name} b={b} entry {j0 + e}: {np.max(err):.3e}"
                n += 1
    assert n == w.B, n


FP8_MAIN = [
    # name, workload, overrides: a token-wise fp8 main cache read by the
    # decode attention and written by the decode prologue's compressor
    ("c4a_decode_B3_L3000", configs.C4A_DECODE_64K, dict(B=3, L=3000)),
    # enough visible entries (9998) for the candidate Top-k, so the prologue
    # (writing the fp8 entry that completes at this step) rides in the
    # indexer's launch
    ("c4a_decode_B2_L40000_fused", configs.C4A_DECODE_64K, dict(B=2, L=40000)),
    ("c4a_decode_L20_tiny", configs.C4A_DECODE_64K, dict(B=2, L=20)),
    ("c128a_L5120", configs.C128A_DECODE_1M, dict(B=2, L=5120, k=64)),
]


@pytest.mark.parametrize("case", FP8_MAIN, ids=[c[0] for c in FP8_MAIN])
def test_layer_decode_fp8_main_cache(case):
    """Decode over a token-wise fp8 main cache: outputs against the oracle
    reading the same codes and scales, and the entry the step completes
    stored as the oracle's quantisation of it (within half a grid step)."""
    name, w0, over = case
    w = configs.shrink(w0, main_cache_dtype="fp8", **over)
    seed = 5700 + FP8_MAIN.index(case)
    print(f"[dsa_layer fp8 main cache] {name} B={w.B} L={w.L} seed={seed}", flush=True)
    inp = gen.layer_inputs(w, seed=seed, state="random")
    st, out, lse, idx = _run_gpu(w, inp)
    ores = _oracle(w, inp, gpu_idx=idx)
    _compare(w, inp, ores, out, lse, idx, label=name)
    codes, sc = st.main_cache.cpu().numpy(), st.main_scale.cpu().numpy()
    n = 0
    for b in range(w.B):
        for j0, n_new, main_new, _ in ores["states"][b].entries_written:
            for e in range(n_new):
                j = j0 + e
                check_fp8_heads(codes[b, j][None], sc[b, j][None], main_new[e][None], 1e-4,
                                f"{name} b={b} entry {j}")
                n += 1
    if (w.L - w.S) % w.s == 0 and w.L >= w.S:
        assert n == w.B, n


# ------------------------------------------------------ rotation offset
OFFSET = 123457


def _split(inp, n_pre, w):
    """The inputs of one token stream cut into a chunk of n_pre tokens and
    the decode step that follows it."""
    pre, dec = dict(inp), dict(inp)
    j_pre = odsa.n_complete(inp["p0"] + n_pre, w.s, w.S) - inp["j0"]
    for key in ("x", "kx", "q", "qi", "qi_scale", "wt"):
        if inp[key] is not None:
            pre[key] = inp[key][:, :n_pre]
            dec[key] = inp[key][:, n_pre:n_pre + 1]
    for key in ("logits_main", "logits_idx"):
        if inp[key] is not None:
            pre[key] = inp[key][:, :j_pre]
            dec[key] = inp[key][:, j_pre:]
    pre.update(T=n_pre, n_new=j_pre)
    dec.update(p0=inp["p0"] + n_pre, T=1, j0=inp["j0"] + j_pre, n_new=inp["n_new"] - j_pre)
    return pre, dec


def test_layer_rope_pos_offset_fresh_sequence():
    """A fresh sequence, so every stored vector is made by the layer: a
    299-token prefill chunk, then the decode step at 299 (which completes an
    entry), with every rotation position shifted by 123,457.  Each step
    against the oracle run with the same shift, and the shifted GPU run
    against the unshifted one: the output depends on relative positions only
    ("DeepSeek V4 稀疏注意力完全解剖", 深潜: Inverse RoPE).  The two GPU runs
    store their rotated vectors in bf16 at different angles, so they agree
    to within that storage rounding (the attention bound, and 1e-2 for the
    log-sum-exp), not bit for bit."""
    w = configs.shrink(configs.C4A_PREFILL_128K, L=300)
    wd = configs.shrink(w, mode="decode")
    inp = gen.layer_inputs(w, seed=5200, p0=0, T=300, state="empty")
    pre, dec = _split(inp, 299, w)
    Ly = _layer()
    res = {}
    for off in (0, OFFSET):
        print(f"[dsa_layer offset] fresh prefill 0..298 + decode 299, offset {off}", flush=True)
        st = Ly.state_from_inputs(inp, DEV)
        _, o1, l1, i1 = _run_gpu(w, pre, state=st, pos_offset=off)
        _, o2, l2, i2 = _run_gpu(wd, dec, state=st, pos_offset=off)
        res[off] = ((o1, l1, i1), (o2, l2, i2))
    # against the oracle with the offset: the chunk, then the decode step
    (o1, l1, i1), (o2, l2, i2) = res[OFFSET]
    g = geometry(w, pos_offset=OFFSET)
    ores = run_layer(g, inp, alt_idx=np.concatenate(
        [i1.cpu().numpy(), i2.cpu().numpy()], axis=1).astype(np.int64))
    ores["qi_dec"] = [decode_store(inp["qi"][b], q_dtype_idx(w.idx_dtype), inp["qi_scale"][b])
                      for b in range(w.B)]
    out = torch.cat([o1, o2], dim=1)
    lse = torch.cat([l1, l2], dim=1)
    idx = torch.cat([i1, i2], dim=1)
    _compare(w, inp, ores, out, lse, idx, label="offset fresh")
    # shifted against unshifted
    for (a, b_) in zip(res[0], res[OFFSET]):
        assert np.array_equal(a[2].cpu().numpy(), b_[2].cpu().numpy()), "selection moved"
        check_close(to_np(b_[0]), to_np(a[0]), ATOL["bf16"], "offset vs none: out")
        check_close(b_[1].cpu().numpy(), a[1].cpu().numpy(), 1e-2, "offset vs none: lse")


def test_layer_rope_pos_offset_decode_random_state():
    """A decode step (completing an entry) with the rotation offset, over a
    random earlier state: against the oracle run with the same offset."""
    w = configs.shrink(configs.C4A_DECODE_64K, B=3, L=3000)
    inp = gen.layer_inputs(w, seed=5201, state="random")
    print(f"[dsa_layer offset] decode B=3 L=3000 offset {OFFSET}", flush=True)
    _, out, lse, idx = _run_gpu(w, inp, pos_offset=OFFSET)
    ores = _oracle(w, inp, gpu_idx=idx, pos_offset=OFFSET)
    _compare(w, inp, ores, out, lse, idx, label="offset decode")


def test_layer_rope_pos_offset_prefill_random_state():
    """A ragged prefill chunk (77 tokens at 2000) with the rotation offset,
    over a random earlier state: against the oracle run with the offset."""
    w = configs.shrink(configs.C4A_PREFILL_128K, L=2077, k=64)
    inp = gen.layer_inputs(w, seed=5202, p0=2000, T=77, state="random")
    print(f"[dsa_layer offset] prefill 2000..2076 offset {OFFSET}", flush=True)
    _, out, lse, idx = _run_gpu(w, inp, pos_offset=OFFSET)
    ores = _oracle(w, inp, gpu_idx=idx, pos_offset=OFFSET)
    _compare(w, inp, ores, out, lse, idx, label="offset prefill")


def test_layer_decode_all_scores_tie():
    """A decode step whose indexer query is zero, so every visible entry
    scores 0: on the candidate path no wave threshold admits a candidate,
    and the attention launch takes the row's cut from the whole row scored
    exactly.  The Top-k is the k lowest indices (ties to the lower index)."""
    w = configs.shrink(configs.C4A_DECODE_64K, B=2, L=40000)
    inp = gen.layer_inputs(w, seed=5800, state="random")
    inp["qi"] = np.zeros_like(inp["qi"])
    print(f"[dsa_layer ties] zero indexer query, B={w.B} L={w.L}", flush=True)
    _, out, lse, idx = _run_gpu(w, inp)
    ix = idx.cpu().numpy()
    for b in range(w.B):
        assert sorted(ix[b, 0].tolist()) == list(range(w.k)), b
    ores = _oracle(w, inp, gpu_idx=idx)
    _compare(w, inp, ores, out, lse, idx, label="all scores tie")


QNORM = [
    # name, workload, overrides, p0, T, state: the Q-norm in the decode
    # prologue riding in the indexer's launch (L = 40000: the candidate
    # path), in the stand-alone prologue (L = 3000, c128a), and in the
    # prefill chunk's pre-attention launch (matrix-core and f32 attention)
    ("c4a_decode_B2_L40000_fused", configs.C4A_DECODE_64K, dict(B=2, L=40000), None, None,
     "random"),
    ("c4a_decode_B3_L3000", configs.C4A_DECODE_64K, dict(B=3, L=3000), None, None, "random"),
    ("c128a_decode_B2_L5000", configs.C128A_DECODE_1M, dict(B=2, L=5000, k=64), None, None,
     "random"),
    ("c4a_prefill_ragged_T77", configs.C4A_PREFILL_128K, dict(L=2077), 2000, 77, "random"),
    ("f32_prefill_fresh_T200", configs.TINY_C4A_F32, dict(L=200, mode="prefill"), 0, 200,
     "empty"),
    # MXFP4 indexer cache: a decode step completing an entry (stand-alone
    # prologue), the same with the prologue in the indexer's launch, and a
    # ragged prefill chunk
    ("c4a_decode_fp4_B3_L3000", configs.C4A_DECODE_1M_FP4, dict(B=3, L=3000), None, None,
     "random"),
    ("c4a_decode_fp4_B2_L40000_fused", configs.C4A_DECODE_1M_FP4, dict(B=2, L=40000), None,
     None, "random"),
    ("c4a_prefill_fp4_ragged_T77", configs.C4A_PREFILL_128K, dict(L=2077, idx_dtype="fp4"),
     2000, 77, "random"),
]


@pytest.mark.parametrize("case", QNORM, ids=[c[0] for c in QNORM])
def test_layer_q_norm(case):
    """Each query head RMS-normalised (gamma per dim) before its rotation,
    prepared in the same launch as the window tokens' rotation ("DeepSeek V4
    稀疏注意力完全解剖", 融合点 3): against the oracle with the same Q-norm."""
    name, w0, over, p0, T, state = case
    w = configs.shrink(w0, **over)
    seed = 5900 + QNORM.index(case)
    print(f"[dsa_layer q-norm] {name} B={w.B} p0={p0} T={T} seed={seed}", flush=True)
    inp = gen.layer_inputs(w, seed=seed, p0=p0, T=T, state=state)
    gam = (1.0 + 0.5 * np.random.default_rng(seed).standard_normal(w.D)).astype(np.float32)
    _, out, lse, idx = _run_gpu(w, inp, q_norm_gamma=torch.tensor(gam, device=DEV))
    ores = _oracle(w, inp, gpu_idx=idx, q_gamma=gam.astype(np.float64))
    _compare(w, inp, ores, out, lse, idx, label=name + " q-norm")
