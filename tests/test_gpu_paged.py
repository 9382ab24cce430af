"""GPU parity of the paged cache layout ("DeepSeek V4 稀疏注意力完全解剖",
第三层 设计 1 and 设计 2; "DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解"
6.1 and 6.2): a logical block is 256 raw positions, so a c4a block holds 64
compressed entries (c128a: 2), the window pool 256 tokens per block, and a
sequence's compressor rings are one block of the ring pools.

Each case runs the same layer step twice from the same seeded inputs: on the
dense per-sequence state and on a paged copy of it whose blocks are scattered
over the pools in a seeded random order (with spare blocks in between).  The
paged run must select the same entries, give the same outputs up to the
summation order (the Top-k pass lists its selection in no fixed order), and
leave the same state behind bit for bit once gathered back through the
tables; every paged output is also checked against the oracle.  Covered: the
decode step with its prologue stand-alone and riding in the indexer's launch,
fp8 and MXFP4 indexer keys, a token-wise fp8 main cache, c128a (2 entries
per block), a ragged prefill chunk, a chunk large enough for the many-rows
indexer contraction (which reads a dense copy of the paged keys), and a block
id outside its pool (reported in the status word, every access kept inside
the pools)."""

import numpy as np
import pytest
import torch

from sparse_long_context_c4a_amd import configs, inputs as gen

from gpu_helpers import ATOL, LSE_ATOL, check_close, to_np
from test_gpu_layer import _compare, _oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, workload, overrides, p0, T
    ("c4a_decode_B3_L3000", configs.C4A_DECODE_64K, dict(B=3, L=3000), None, None),
    ("c4a_decode_B2_L40000_fused", configs.C4A_DECODE_64K, dict(B=2, L=40000), None, None),
    ("c4a_decode_fp4_B2_L40000_fused", configs.C4A_DECODE_1M_FP4, dict(B=2, L=40000), None,
     None),
    ("c4a_decode_fp8_main_B2_L40000", configs.C4A_DECODE_64K,
     dict(B=2, L=40000, main_cache_dtype="fp8"), None, None),
    ("c128a_decode_B2_L5120", configs.C128A_DECODE_1M, dict(B=2, L=5120, k=64), None, None),
    ("c4a_prefill_ragged_T77", configs.C4A_PREFILL_128K, dict(L=2077), 2000, 77),
    ("c4a_prefill_contraction_B2_T300", configs.C4A_PREFILL_128K, dict(B=2, L=4300), 4000, 300),
    # MXFP4 keys: the chunk's two compressions in one launch, both paged
    ("c4a_prefill_fp4_ragged_T77", configs.C4A_PREFILL_128K, dict(L=2077, idx_dtype="fp4"), 2000,
     77),
    ("c128a_prefill_T300", configs.C128A_DECODE_1M, dict(B=2, L=1300, k=64, mode="prefill"), 1000,
     300),
]


def _run(Ly, w, st, inp, pages=None):
    ch = Ly.chunk_from_inputs(w, inp, DEV)
    out, lse, idx, status, _ = Ly.run(w, st, ch, max_pos_end=st.e_cap * w.s, pages=pages)
    torch.cuda.synchronize()
    return out, lse, idx, status.item()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_layer_matches_dense(case):
    from sparse_long_context_c4a_amd import layer as Ly
    name, w0, over, p0, T = case
    w = configs.shrink(w0, **over)
    seed = 8100 + CASES.index(case)
    inp = gen.layer_inputs(w, seed=seed, p0=p0, T=T, state="random")
    p0, T = inp["p0"], inp["T"]
    print(f"[dsa_layer paged] {name} B={w.B} p0={p0} T={T} seed={seed}", flush=True)
    st = Ly.state_from_inputs(inp, DEV)
    pst, pages = Ly.page_state(w, Ly.state_from_inputs(inp, DEV), p0, seed=seed)
    out, lse, idx, s0 = _run(Ly, w, st, inp)
    pout, plse, pidx, s1 = _run(Ly, w, pst, inp, pages)
    assert s0 == 0 and s1 == 0, (s0, s1)
    # the same selection, outputs up to the summation order
    gi, pi = idx.cpu().numpy(), pidx.cpu().numpy()
    for b in range(w.B):
        for t in range(T):
            assert set(gi[b, t].tolist()) == set(pi[b, t].tolist()), f"{name} b={b} t={t}"
    check_close(to_np(pout), to_np(out), ATOL[w.main_dtype], f"{name} paged vs dense out")
    check_close(plse.cpu().numpy(), lse.cpu().numpy(), LSE_ATOL[w.main_dtype],
                f"{name} paged vs dense lse")
    # the state left behind, gathered back through the tables
    dense = Ly.unpage_state(w, pst, pages, st)
    assert torch.equal(dense["main_cache"], st.main_cache), "main cache"
    if st.main_scale is not None:
        assert torch.equal(dense["main_scale"], st.main_scale), "main scales"
    if st.idx_cache is not None:
        assert torch.equal(dense["idx_cache"], st.idx_cache), "indexer keys"
        for f in ("idx_scale", "idx_mx"):
            if getattr(st, f) is not None:
                assert torch.equal(dense[f], getattr(st, f)), f
    assert torch.equal(dense["main_ring"], st.main_ring), "main ring"
    if st.idx_ring is not None:
        assert torch.equal(dense["idx_ring"], st.idx_ring), "indexer ring"
    lo = max(0, p0 + T - w.W)
    assert torch.equal(Ly.unpage_window(pst, pages, lo, p0 + T),
                       Ly.dense_window(st, lo, p0 + T)), "window tokens"
    # and the paged outputs against the oracle (all rows of a decode step,
    # up to 64 spread rows of a chunk)
    rows = None if T == 1 else sorted(set(np.linspace(0, T - 1, 64).astype(int).tolist()))
    ores = _oracle(w, inp, only=rows, gpu_idx=pidx)
    _compare(w, inp, ores, pout, plse, pidx, rows=rows, label=f"{name} paged")


def test_paged_block_outside_pool_is_reported():
    """A table entry naming a block beyond the pool, for an entry the step
    reads: DSA_DEVERR_BLOCK in the status word and no access outside the
    pools (the read goes to block 0)."""
    from sparse_long_context_c4a_amd import _lib
    from sparse_long_context_c4a_amd import layer as Ly
    w = configs.shrink(configs.C4A_DECODE_64K, B=2, L=40000)
    inp = gen.layer_inputs(w, seed=8200, state="random")
    print(f"[dsa_layer paged] block id beyond the pool, B={w.B} L={w.L}", flush=True)
    pst, pages = Ly.page_state(w, Ly.state_from_inputs(inp, DEV), inp["p0"], seed=8200)
    pages.table[1, 3] = pages.n_blocks + 5   # entries 192 .. 255 of sequence 1
    _, _, _, status = _run(Ly, w, pst, inp, pages)
    assert status & _lib.DEVERR_BLOCK, status
