"""dsa_layer_decode_noalloc -- the decode step for callers that cannot
allocate, on the library's static scratch -- against dsa_layer_decode with
a caller's workspace.  Two calls in a row on one GPU, the second with a
smaller input (a different geometry, so the scratch holds the first call's
leftovers), each entry point on its own copy of the same state: outputs,
log-sum-exps, selections and the state the step leaves behind must agree
(to the attention bound; the kernels are the same, so in practice bit for
bit)."""

import numpy as np
import pytest
import torch

from sparse_long_context_c4a_amd import configs, inputs as gen

from gpu_helpers import ATOL, LSE_ATOL, check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # a large scratch first (c128a at 1M: 18 MiB), then a smaller c4a step
    # whose Top-k runs on the candidate path
    ("c128a_decode_B16_L1M", configs.C128A_DECODE_1M, {}),
    ("c4a_decode_B2_L40000", configs.C4A_DECODE_64K, dict(B=2, L=40000)),
]


def _state_tensors(st):
    return [t for t in (st.main_cache, st.idx_cache, st.idx_scale, st.main_ring, st.idx_ring,
                        st.window, st.main_scale) if t is not None]


def test_noalloc_decode_matches_workspace_decode_twice():
    from sparse_long_context_c4a_amd import _lib
    from sparse_long_context_c4a_amd import layer as Ly
    cap = _lib.layer_decode_noalloc_capacity()
    for i, (name, w0, over) in enumerate(CASES):
        w = configs.shrink(w0, **over)
        print(f"[dsa_layer_decode_noalloc] call {i + 1}: {name} B={w.B} L={w.L}", flush=True)
        inp = gen.layer_inputs(w, seed=7300 + i)
        st_a, st_b = Ly.state_from_inputs(inp, DEV), Ly.state_from_inputs(inp, DEV)
        ch = Ly.chunk_from_inputs(w, inp, DEV)
        del inp
        # the existing entry point with a workspace
        out_a, lse_a, idx_a, status_a, ws = Ly.run(w, st_a, ch, max_pos_end=st_a.e_cap * w.s)
        # the allocation-free one
        out_b, lse_b, idx_b, status_b = Ly.alloc_outputs(w, w.B, 1, DEV)
        a = Ly.layer_args(w, st_b, ch, out_b, lse_b, idx_b, status_b,
                          max_pos_end=st_b.e_cap * w.s)
        assert _lib.layer_workspace(a) <= cap
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        _lib.layer_decode_noalloc(a)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert status_a.item() == 0 and status_b.item() == 0
        ia, ib = idx_a.cpu().numpy(), idx_b.cpu().numpy()
        for b in range(w.B):
            assert set(ia[b, 0].tolist()) == set(ib[b, 0].tolist()), f"{name} b={b} selection"
        err = check_close(to_np(out_b), to_np(out_a), ATOL[w.main_dtype], f"{name} out")
        check_close(lse_b.cpu().numpy(), lse_a.cpu().numpy(), LSE_ATOL[w.main_dtype], f"{name} lse")
        print(f"[dsa_layer_decode_noalloc] {name}: max |out diff| {err:.3e}", flush=True)
        for ta, tb in zip(_state_tensors(st_a), _state_tensors(st_b)):
            assert torch.equal(ta, tb), f"{name}: state differs"
        del ws, st_a, st_b, ch
        torch.cuda.empty_cache()
