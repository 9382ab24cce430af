"""Benchmark of the compressed sparse attention layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one dsa_layer_decode call over one batch (compress the entry that
completes at m, index every visible entry, Top-k, sparse attention, window
insert) on seeded synthetic inputs already resident in HBM.  Input sets are
rotated (three by default) so that repeated steps do not find the indexer
keys in the 256 MB Infinity Cache.  Prints one JSON line: the headline c4a
decode (B=4, L=1M) as the value, the prefill chunk under "prefill", the
other decode workloads under "workloads" (--no-extra skips them; there also
the headline step with its output stored as fp8) and the oracle's rate on a
bounded sample under "cpu_baseline".
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "c4a DSA decode queries/s + HBM GB/s (% peak) at L=1M k=512; prefill TFLOP/s"
PEAK_HBM_GBPS = 8000.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_BF16_TFLOPS = 2500.0
# KV-cache sizes the pages print for whole models at 1M tokens ("DeepSeek V4
# 稀疏注意力完全解剖", opening table: 61 layers), reported beside the
# throughput as context only -- they are memory sizes, not kernel timings.
PAGE_KV_CONTEXT = {
    "source": "DeepSeek V4 稀疏注意力完全解剖, opening table (61 layers, 1M-token sequence)",
    "kv_gib_per_seq": {"V3.2": 83.9, "V4 bf16": 9.62, "V4 fp4 indexer + fp8 attention": 4.8},
    "kv_bytes_per_token_per_layer": {"V3.2": 1408, "V4 bf16 (average over layers)": 160,
                                     "V4 fp4 indexer + fp8 attention (average)": 80},
}


# Hardware byte counters of the scoring kernel, from the committed rocprofv3
# summary; reported only while the sources they were taken from are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_decode_index_c4a_decode_B4_L1M.txt")
TRAFFIC_SOURCES = ["indexer.hip", "indexer_impl.h", "select_impl.h", "decode_impl.h",
                   "compress_impl.h", "common.h", "internal.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_long_context_c4a_amd", "csrc")
    for f in TRAFFIC_SOURCES + ["../../include/dsa.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, each scaled by the
    copy calibration) from the summary file, or None if it is missing or was
    taken from other kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith(" "):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_hash") != kernel_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def index_key_bytes(w):
    """Bytes of one stored indexer key with its scales."""
    if not w.Hi:
        return 0
    return {"fp8": w.Di + 4, "fp4": w.Di // 2 + w.Di // 32, "f32": 4 * w.Di}[w.idx_dtype]


def decode_bytes_per_query(w, nv):
    """Algorithmic HBM bytes of one decode query: the visible indexer keys
    (fp8: Di bytes + a 4-byte scale each; MXFP4: Di / 2 bytes + Di / 32
    scale bytes), the k + W gathered latent vectors, q and out, and the k
    selected indices."""
    el = 2 if w.main_dtype == "bf16" else 4
    idx_b = nv * index_key_bytes(w)
    sel = min(w.k, nv)
    attn = (sel + min(w.W, w.m)) * w.D * el
    return idx_b + attn + 2 * w.H * w.D * el + w.k * 4


def build_sets(w, n_sets, device):
    from sparse_long_context_c4a_amd import inputs as gen
    from sparse_long_context_c4a_amd import layer as Ly
    sets = []
    for i in range(n_sets):
        inp = gen.layer_inputs(w, seed=w.seed + 1000 * i)
        st = Ly.state_from_inputs(inp, device)
        ch = Ly.chunk_from_inputs(w, inp, device)
        sets.append((st, ch))
        del inp
    return sets


def time_layer(w, sets, steps, warmup, decode, out_fp8=False, q_norm=False):
    """Two timed passes after `warmup` untimed steps.  The first, of `steps`
    steps, gives the step time: nothing but the layer's own launches on the
    stream, bracketed by events.  The second (`steps` steps, at least 100 for
    decode) hands the library HIP events (dsa_set_timing_events) that it
    attaches to the dispatch packets of the scoring kernel and of the
    attention kernels (hipExtLaunchKernel), which gives their own mean
    durations on the stream they run on.  With out_fp8 the layer stores its
    output as fp8 codes with one scale per (row, head)."""
    import torch
    from sparse_long_context_c4a_amd import _lib
    from sparse_long_context_c4a_amd import layer as Ly
    dev = sets[0][1].x.device
    B, T = sets[0][1].x.shape[0], sets[0][1].T
    outs = [Ly.alloc_outputs(w, B, T, dev, out_fp8) for _ in sets]
    scs = [torch.empty((B, T, w.H), dtype=torch.float32, device=dev) if out_fp8 else None
           for _ in sets]
    qg = None
    if q_norm:  # a Q-norm weight around 1
        g = torch.Generator(device="cpu").manual_seed(5)
        qg = (1.0 + 0.5 * torch.randn(w.D, generator=g)).to(dev)
    # a set is (state, chunk) or, paged, (pool state, chunk, block tables)
    args = [Ly.layer_args(w, s[0], s[1], *o, max_pos_end=s[0].e_cap * w.s, out_scale=sc,
                          q_norm_gamma=qg, pages=s[2] if len(s) > 2 else None)
            for s, o, sc in zip(sets, outs, scs)]
    ws_bytes = max(_lib.layer_workspace(a) for a in args)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fn = _lib.layer_decode if decode else _lib.layer_prefill
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(args[i % len(args)], ws=ws, stream=stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        fn(args[i % len(args)], ws=ws, stream=stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    # the kernel durations: a mean over at least 100 consecutive steps (a
    # mean over 20 moved by +-1.5 us between runs at the headline workload;
    # over 100 it holds within a few tenths)
    n_ev = max(steps, 100) if decode else steps
    ev_i = [(_lib.HipEvent(), _lib.HipEvent()) for _ in range(n_ev)]
    ev_a = [(_lib.HipEvent(), _lib.HipEvent()) for _ in range(n_ev)]
    for i in range(n_ev):
        _lib.set_timing_events(index=ev_i[i], attn=ev_a[i])
        fn(args[i % len(args)], ws=ws, stream=stream)
    torch.cuda.synchronize()
    st = [o[3].item() for o in outs]
    assert all(s == 0 for s in st), f"device status {st}"
    # (a workload without an indexer, k >= every n_vis, never records the
    # indexer's events)
    idx_ms = sum(e[0].elapsed_ms(e[1]) for e in ev_i) / n_ev if w.Hi else None
    attn_ms = sum(e[0].elapsed_ms(e[1]) for e in ev_a) / n_ev
    return ms, idx_ms, attn_ms


def time_layer_graph(w, sets, steps, warmup):
    """The decode step captured once per input set in a HIP graph
    (torch.cuda.CUDAGraph over the library's launches) and replayed round
    robin over the sets: the step time without per-launch host work.  A
    replay repeats its set's step at the same positions, which rewrites the
    same state values, so the replays are equivalent to the eager steps."""
    import torch
    from sparse_long_context_c4a_amd import _lib
    from sparse_long_context_c4a_amd import layer as Ly
    dev = sets[0][1].x.device
    B = sets[0][1].x.shape[0]
    outs = [Ly.alloc_outputs(w, B, 1, dev) for _ in sets]
    args = [Ly.layer_args(w, st, ch, *o, max_pos_end=st.e_cap * w.s)
            for (st, ch), o in zip(sets, outs)]
    ws = torch.empty(max(_lib.layer_workspace(a) for a in args), dtype=torch.uint8, device=dev)
    graphs = []
    for a in args:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _lib.layer_decode(a, ws=ws, stream=torch.cuda.current_stream())
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    t1.record(stream)
    torch.cuda.synchronize()
    assert all(o[3].item() == 0 for o in outs)
    del graphs
    return t0.elapsed_time(t1) / steps


def cpu_baseline(w, min_seconds=10.0, max_sets=8):
    """The fp64 oracle on a bounded sample of the same workload: full layer
    steps for all w.B decode queries of successive seeded input sets, until
    at least min_seconds of oracle time (or max_sets sets) have been spent.
    Input generation is outside the timed part."""
    from threadpoolctl import threadpool_info

    from oracle.layer import Geometry
    from oracle.run import run_layer
    from sparse_long_context_c4a_amd import inputs as gen
    g = Geometry(s=w.s, S=w.S, D=w.D, r=w.r, Di=w.Di, r_idx=w.r_idx, H=w.H, Hi=w.Hi, k=w.k,
                 W=w.W, main_dtype=w.main_dtype, idx_dtype=w.idx_dtype)
    dt, n = 0.0, 0
    for i in range(max_sets):
        inp = gen.layer_inputs(w, seed=w.seed + 1000 * i)
        t = time.perf_counter()
        run_layer(g, inp)
        dt += time.perf_counter() - t
        n += w.B
        del inp
        if dt >= min_seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": n / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} decode queries of {w.name} ({n // w.B} seeded input sets of "
                      f"{w.B}; full layer step, fp64 NumPy), {dt:.1f} s of oracle time"}


def time_attn_cache(w, dev, fp8_cache, steps=200, warmup=20):
    """The attention op alone (dsa_sparse_attn) at a decode workload's shapes
    -- B rows at m = L - 1, k selected entries among the visible ones, the
    W-token window -- over a bf16 cache or a token-wise fp8 one (codes and
    one scale per entry, the window bf16).  Random bits drawn on the GPU."""
    import torch
    from sparse_long_context_c4a_amd import _lib
    torch.manual_seed(7)
    nv = _lib.n_complete(w.m, w.s, w.S)
    e_cap = nv + 2
    if fp8_cache:  # e4m3fn codes without the NaN patterns, scales in [0.5, 1.5)
        cache = (torch.randint(0, 0x7f, (w.B, e_cap, w.D), dtype=torch.uint8, device=dev) |
                 (torch.randint(0, 2, (w.B, e_cap, w.D), dtype=torch.uint8, device=dev) << 7))
        csc = torch.rand((w.B, e_cap), device=dev) + 0.5
    else:
        cache = torch.randn((w.B, e_cap, w.D), device=dev, dtype=torch.bfloat16)
        csc = None
    win = torch.randn((w.B, w.W, w.D), device=dev, dtype=torch.bfloat16)
    q = torch.randn((w.B, w.H, w.D), device=dev, dtype=torch.bfloat16)
    idx = torch.stack([torch.randperm(nv, device=dev)[:w.k] for _ in range(w.B)]).to(torch.int32)
    qpos = torch.full((w.B,), w.m, dtype=torch.int64, device=dev)
    out = torch.empty((w.B, w.H, w.D), device=dev, dtype=torch.bfloat16)
    a = _lib.AttnArgs()
    a.n_seqs, a.queries_per_seq, a.q_pos, a.heads, a.dim = w.B, 1, _lib.ptr(qpos), w.H, w.D
    a.rope_dim, a.rope_base, a.rope_pos_offset = w.r, w.base, 0
    a.dtype, a.q, a.rotate_q = _lib.DSA_BF16, _lib.ptr(q), 1
    a.cache, a.e_cap, a.idx, a.k = _lib.ptr(cache), e_cap, _lib.ptr(idx), w.k
    a.window, a.w_cap, a.window_size = _lib.ptr(win), w.W, w.W
    a.softmax_scale, a.max_pos_end, a.out = 0.0, w.m + 1, _lib.ptr(out)
    if fp8_cache:
        a.cache_fp8, a.cache_scale = 1, _lib.ptr(csc)
    ws = _lib.sparse_attn(a)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        _lib.sparse_attn(a, ws=ws, stream=stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        _lib.sparse_attn(a, ws=ws, stream=stream)
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / steps * 1e3
    el = 1 if fp8_cache else 2
    gathered = w.B * (w.k * w.D * el + w.W * w.D * 2)
    del cache, csc
    torch.cuda.empty_cache()
    return {"us_per_call": us, "cache": "fp8 token-wise" if fp8_cache else "bf16",
            "gathered_bytes": gathered, "rows": w.B, "k": w.k, "window": w.W}


READ_PROBE = os.path.join(ROOT, "tests", "hw", "libhbm_read_probe.so")


def time_plain_read(dev, total_bytes, n_wg, steps=20, warmup=5):
    """A plain streaming read of about `total_bytes` (rounded up to 16-byte
    pieces per workgroup) over n_wg workgroups of 256 threads, timed like
    the indexer (events on its own dispatch packets), as the practical
    read rate of one launch of that size.  The source is 1 GiB read in
    rotating spans so that no launch finds its span in the Infinity Cache.
    None when the probe library is not built."""
    import ctypes
    import torch
    from sparse_long_context_c4a_amd import _lib
    if not os.path.exists(READ_PROBE):
        return None
    lib = ctypes.CDLL(READ_PROBE)
    lib.hbm_read_probe.restype = ctypes.c_int
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]
    per = -(-total_bytes // (16 * n_wg)) * 16
    src_bytes = 1 << 30
    spans = src_bytes // (per * n_wg)
    assert spans >= 4, "span too large for the rotation"
    src = torch.ones(src_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(n_wg, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    evs = [(_lib.HipEvent(), _lib.HipEvent()) for _ in range(steps)]
    for i in range(warmup + steps):
        e0, e1 = evs[i - warmup] if i >= warmup else (None, None)
        off = (i % spans) * per * n_wg
        rc = lib.hbm_read_probe(src.data_ptr() + off, src_bytes - off, per, n_wg,
                                sink.data_ptr(), stream, e0.handle if e0 else None,
                                e1.handle if e1 else None)
        assert rc == 0, f"hbm_read_probe returned {rc}"
    torch.cuda.synchronize()
    us = sum(e[0].elapsed_ms(e[1]) for e in evs) / steps * 1e3
    del src, sink
    return {"kernel": "plain streaming read (tests/hw/hbm_read_probe.hip)", "bytes": per * n_wg,
            "workgroups": n_wg, "us": us, "gbps": per * n_wg / (us * 1e-6) / 1e9}


def time_prefill(dev, steps=3, warmup=1):
    """The prefill chunk workload: layer step time, indexer (+Top-k) and
    attention kernel times, and their throughput."""
    import torch
    from sparse_long_context_c4a_amd import configs, _lib
    wp = configs.C4A_PREFILL_128K
    print("[bench] prefill chunk", file=sys.stderr, flush=True)
    psets = build_sets(wp, 1, dev)
    pms, pidx_ms, pattn_ms = time_layer(wp, psets, steps, warmup, decode=False)
    nvs = sum(_lib.n_complete(wp.p0 + t, wp.s, wp.S) for t in range(wp.T))
    idx_flop = 2.0 * wp.Hi * wp.Di * nvs
    attn_flop = 4.0 * wp.T * wp.H * (wp.k + wp.W) * wp.D
    del psets
    torch.cuda.empty_cache()
    return {"workload": wp.name, "ms_per_step": pms,
            "indexer_ms": pidx_ms, "attention_ms": pattn_ms,
            "indexer_tflops": idx_flop / (pidx_ms / 1e3) / 1e12,
            "indexer_frac_fp8_peak": idx_flop / (pidx_ms / 1e3) / 1e12 / PEAK_FP8_TFLOPS,
            "attention_tflops": attn_flop / (pattn_ms / 1e3) / 1e12,
            "attention_frac_bf16_peak": attn_flop / (pattn_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "layer_tflops": (idx_flop + attn_flop) / (pms / 1e3) / 1e12}


def time_decode_workload(w, dev, steps, warmup, n_sets):
    """Step time and throughput of one more decode workload (reported beside
    the headline; each is also a parity-test case)."""
    import torch
    from sparse_long_context_c4a_amd import _lib
    print(f"[bench] decode workload {w.name}", file=sys.stderr, flush=True)
    sets = build_sets(w, n_sets, dev)
    ms, idx_ms, attn_ms = time_layer(w, sets, steps, warmup, decode=True)
    del sets
    torch.cuda.empty_cache()
    nv = _lib.n_complete(w.m, w.s, w.S)
    step_bytes = w.B * decode_bytes_per_query(w, nv)
    gbps = step_bytes / (ms / 1e3) / 1e9
    r = {"queries_per_s": w.B / (ms / 1e3), "ms_per_step": ms, "batch": w.B, "context": w.L,
         "k": w.k, "n_vis": nv, "alg_bytes_per_step": step_bytes, "hbm_gbps": gbps,
         "hbm_frac": gbps / PEAK_HBM_GBPS,
         "kernel_ms": {"indexer": idx_ms, "attention": attn_ms}}
    if w.Hi and idx_ms:  # the key stream's own rate (keys and their scales)
        r["indexer_key_bytes"] = index_key_bytes(w)
        r["indexer_gbps"] = w.B * nv * index_key_bytes(w) / (idx_ms / 1e3) / 1e9
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4a_decode_B4_L1M")
    ap.add_argument("--sets", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other decode workloads (reported under 'workloads')")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill chunk (for profiling its kernels)")
    ap.add_argument("--print-source-hash", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB three times "
                         "(a known-size reference for hardware byte counters)")
    args = ap.parse_args()
    if args.print_source_hash:
        print(kernel_source_hash())
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the layer's multi-GPU "
              "sharding is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_long_context_c4a_amd import configs
    from sparse_long_context_c4a_amd import _lib
    w = configs.BY_NAME[args.workload]
    assert w.mode == "decode"
    dev = "cuda"
    if args.prefill_only:
        print(json.dumps({"prefill": time_prefill(dev)}))
        return
    print(f"[bench] building {args.sets} input sets for {w.name}", file=sys.stderr, flush=True)
    sets = build_sets(w, args.sets, dev)
    print("[bench] timing", file=sys.stderr, flush=True)
    ms, idx_ms, attn_ms = time_layer(w, sets, args.steps, args.warmup, decode=True)
    nv = _lib.n_complete(w.m, w.s, w.S)
    qps = w.B / (ms / 1e3)
    step_bytes = w.B * decode_bytes_per_query(w, nv)
    gbps = step_bytes / (ms / 1e3) / 1e9
    if w.Hi:
        # the dominant kernel: the indexer's stream over the visible keys
        kern, kbytes, kms = "k_decode_index", w.B * nv * index_key_bytes(w), idx_ms
    else:
        # no indexer (the selection is every visible entry): the attention
        # kernels' gather of the n_vis + W vectors, q and out
        el = 2 if w.main_dtype == "bf16" else 4
        kern = "attention+combine"
        kbytes = w.B * ((min(w.k, nv) + min(w.W, w.m)) * w.D * el + 2 * w.H * w.D * el)
        kms = attn_ms
    kgbps = kbytes / (kms / 1e3) / 1e9 if kms else None
    line = {
        "metric": METRIC, "value": qps, "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "context": w.L, "query_pos": w.m,
                   "n_vis": nv, "k": w.k, "window": w.W, "latent_dim": w.D, "heads": w.H,
                   "indexer_heads": w.Hi, "indexer_dim": w.Di, "input_sets": args.sets},
        "hbm_gbps": gbps, "hbm_frac": gbps / PEAK_HBM_GBPS, "alg_bytes_per_step": step_bytes,
        "kernel_ms": {"indexer": idx_ms, "attention": attn_ms},
        "roofline": {"bound": "hbm", "achieved": kgbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": kgbps / PEAK_HBM_GBPS if kgbps else None,
                     "traffic": measured_traffic() if w.name == "c4a_decode_B4_L1M" else None,
                     "kernel": kern, "alg_bytes_per_launch": kbytes},
    }
    # this layer's own cache per raw token: one main entry (D dims) and one
    # indexer key (with its scales) per s tokens; the window ring
    # is a fixed W tokens per sequence
    el = 2 if w.main_dtype == "bf16" else 4
    ikey = index_key_bytes(w)
    line["kv_context"] = dict(PAGE_KV_CONTEXT, this_layer={
        "layer": w.name.split("_")[0], "bytes_per_token": (w.D * el + ikey) / w.s,
        "window_bytes_per_seq": w.W * w.D * el})
    extra = {}
    if not args.no_extra and w.name == "c4a_decode_B4_L1M":
        # the same step with the output stored as fp8 (scale per row and head)
        print("[bench] timing with fp8 output", file=sys.stderr, flush=True)
        ms8, _, attn8 = time_layer(w, sets, args.steps, args.warmup, decode=True, out_fp8=True)
        extra[w.name + "_fp8_out"] = {"queries_per_s": w.B / (ms8 / 1e3), "ms_per_step": ms8,
                                      "batch": w.B, "context": w.L, "k": w.k,
                                      "kernel_ms": {"attention": attn8}}
        # the same step with a Q-norm of every query head, prepared in the
        # indexer's launch
        print("[bench] timing with a Q-norm", file=sys.stderr, flush=True)
        msq, _, attnq = time_layer(w, sets, args.steps, args.warmup, decode=True, q_norm=True)
        extra[w.name + "_q_norm"] = {"queries_per_s": w.B / (msq / 1e3), "ms_per_step": msq,
                                     "batch": w.B, "context": w.L, "k": w.k,
                                     "kernel_ms": {"attention": attnq}}
        # the same step captured in HIP graphs and replayed
        print("[bench] timing graph replays", file=sys.stderr, flush=True)
        msg = time_layer_graph(w, sets, args.steps, args.warmup)
        extra[w.name + "_graph_replay"] = {"queries_per_s": w.B / (msg / 1e3), "ms_per_step": msg,
                                           "batch": w.B, "context": w.L, "k": w.k}
        # the same step over paged caches (256-position logical blocks, the
        # blocks scattered over the pools in a seeded random order)
        print("[bench] timing over paged caches", file=sys.stderr, flush=True)
        from sparse_long_context_c4a_amd import layer as Ly
        sets_p = []
        for i, (st, ch) in enumerate(sets):
            pst, pages = Ly.page_state(w, st, w.m, seed=i)
            sets_p.append((pst, ch, pages))
        msp, idxp, attnp = time_layer(w, sets_p, args.steps, args.warmup, decode=True)
        del sets_p
        torch.cuda.empty_cache()
        extra[w.name + "_paged"] = {
            "queries_per_s": w.B / (msp / 1e3), "ms_per_step": msp, "batch": w.B,
            "context": w.L, "k": w.k, "entries_per_block": 256 // w.s,
            "kernel_ms": {"indexer": idxp, "attention": attnp}}
        # the same step over a token-wise fp8 main cache (decode prologue
        # unfused, the attention reading fp8 entries)
        print("[bench] timing over an fp8 main cache", file=sys.stderr, flush=True)
        wm = configs.shrink(w, main_cache_dtype="fp8")
        sets_m = build_sets(wm, args.sets, dev)
        msm, idxm, attnm = time_layer(wm, sets_m, args.steps, args.warmup, decode=True)
        del sets_m
        extra[w.name + "_fp8_main_cache"] = {
            "queries_per_s": w.B / (msm / 1e3), "ms_per_step": msm, "batch": w.B,
            "context": w.L, "k": w.k, "kernel_ms": {"indexer": idxm, "attention": attnm}}
    del sets
    torch.cuda.empty_cache()
    if w.Hi and kgbps and not args.no_extra:
        # what a launch that only reads the indexer's bytes, over its grid of
        # stream workgroups (1024 entries each), reaches on this GPU
        print("[bench] plain read of the indexer's bytes", file=sys.stderr, flush=True)
        rd = time_plain_read(dev, kbytes, w.B * (-(-nv // 1024)))
        if rd:
            rd["frac_of_peak"] = rd["gbps"] / PEAK_HBM_GBPS
            rd["indexer_vs_plain_read"] = kgbps / rd["gbps"]
        line["roofline"]["plain_read"] = rd
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calib_copy_bytes"] = n
        del src, dst
    if not args.no_prefill:
        line["prefill"] = time_prefill(dev)
    if not args.no_extra and w.name == "c4a_decode_B4_L1M":
        line["workloads"] = {
            x.name: time_decode_workload(x, dev, args.steps, args.warmup, args.sets)
            for x in configs.ALL if x.mode == "decode" and x.name != w.name}
        line["workloads"].update(extra)
        # the attention op alone over a bf16 and an fp8 cache
        print("[bench] attention op over bf16 and fp8 caches", file=sys.stderr, flush=True)
        line["workloads"]["attn_op_" + w.name] = {
            "bf16_cache": time_attn_cache(w, dev, False),
            "fp8_cache": time_attn_cache(w, dev, True)}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
