"""Resumable state on the GPU.  Between calls the layer keeps nothing of its
own: a sequence's state is its main cache, indexer cache (with scales), the
two compressor rings (the raw tokens of the entry still being filled, which
the pages keep at block boundaries: "DeepSeek V4 稀疏注意力完全解剖", 第三层
设计 2) and the window ring, plus the next position.  So a run resumed from a
copy of that state, taken to host memory and put back in fresh device
allocations, must equal the uninterrupted run: the same selections, the same
outputs (to the attention's summation order: the Top-k may emit a selection
in another order) and the same state afterwards, bit for bit; and the
resumed run's last step matches the oracle run over the whole token stream."""

import pytest
import torch

from oracle import dsa as odsa
from oracle.run import run_layer
from sparse_long_context_c4a_amd import configs, inputs as gen

from gpu_helpers import ATOL, LSE_ATOL, check_close, geometry, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"

STATE_FIELDS = ("main_cache", "idx_cache", "idx_scale", "main_ring", "idx_ring", "window",
                "main_scale", "idx_mx")


def _pieces(inp, sizes, p0):
    """The token stream of `inp` (p0 .. p0 + T - 1) cut into consecutive
    calls of the given sizes."""
    j0 = inp["j0"]
    out, p = [], 0
    for T in sizes:
        sub = dict(inp)
        a, b = odsa.n_complete(p0 + p, 4, 8), odsa.n_complete(p0 + p + T, 4, 8)
        for key in ("x", "kx", "q", "qi", "qi_scale", "wt"):
            if inp.get(key) is not None:
                sub[key] = inp[key][:, p:p + T]
        for key in ("logits_main", "logits_idx"):
            sub[key] = inp[key][:, a - j0:b - j0]
        sub.update(p0=p0 + p, T=T, j0=a, n_new=b - a)
        out.append(sub)
        p += T
    return out


def _step(Ly, w, st, sub):
    ch = Ly.chunk_from_inputs(w, sub, DEV)
    out, lse, idx, status, _ = Ly.run(w, st, ch, decode=(sub["T"] == 1) or None,
                                      max_pos_end=st.e_cap * w.s)
    torch.cuda.synchronize()
    assert status.item() == 0, f"device status {status.item()}"
    return out, lse, idx


def _restored(Ly, st):
    """The state copied to host memory and back into new device tensors."""
    host = {f: (None if getattr(st, f) is None else getattr(st, f).cpu().clone())
            for f in STATE_FIELDS}
    back = {f: (None if t is None else t.to(DEV)) for f, t in host.items()}
    for f in STATE_FIELDS:  # fresh allocations, not views of the originals
        if back[f] is not None:
            assert back[f].data_ptr() != getattr(st, f).data_ptr()
    return Ly.LayerState(e_cap=st.e_cap, **back)


@pytest.mark.parametrize("idx_dtype", ["fp8", "fp4"])
def test_resumed_run_equals_uninterrupted(idx_dtype):
    from sparse_long_context_c4a_amd import layer as Ly
    w = configs.shrink(configs.C4A_PREFILL_128K, L=3064, idx_dtype=idx_dtype)
    p0 = 3000
    inp = gen.layer_inputs(w, seed=5300, p0=p0, T=64, state="random")
    print(f"[dsa_layer] resume {idx_dtype}: chunk 3000..3049, then 3050..3062 and the "
          f"decode step 3063", flush=True)
    first, *rest = _pieces(inp, (50, 13, 1), p0)
    # uninterrupted
    st_a = Ly.state_from_inputs(inp, DEV)
    _step(Ly, w, st_a, first)
    res_a = [_step(Ly, w, st_a, sub) for sub in rest]
    # the same first call, then the state saved, restored, and the run resumed
    st_b = Ly.state_from_inputs(inp, DEV)
    _step(Ly, w, st_b, first)
    st_c = _restored(Ly, st_b)
    del st_b
    res_c = [_step(Ly, w, st_c, sub) for sub in rest]
    for k, ((oa, la, ia), (oc, lc, ic)) in enumerate(zip(res_a, res_c)):
        ia, ic = ia.cpu().numpy(), ic.cpu().numpy()
        for b in range(w.B):
            for t in range(ia.shape[1]):
                assert set(ia[b, t].tolist()) == set(ic[b, t].tolist()), (k, b, t)
        check_close(to_np(oc), to_np(oa), ATOL[w.main_dtype], f"call {k + 2}: out")
        check_close(lc.cpu().numpy(), la.cpu().numpy(), LSE_ATOL[w.main_dtype],
                    f"call {k + 2}: lse")
    for f in STATE_FIELDS:
        ta, tc = getattr(st_a, f), getattr(st_c, f)
        assert (ta is None) == (tc is None), f
        if ta is not None:
            assert torch.equal(ta, tc), f"state {f} differs"
    # the resumed run's decode step against the oracle over the whole stream
    last = p0 + 63
    ores = run_layer(geometry(w), inp, only=[63])
    out, lse, idx = res_c[-1]
    dt = w.main_dtype
    compared = 0
    for b in range(w.B):
        got = set(idx.cpu().numpy()[b, 0].tolist()) - {-1}
        want = set(ores["idx"][b, 63].tolist()) - {-1}
        assert len(got) == len(want) == min(w.k, odsa.n_vis(last, w.s, w.S))
        assert len(got ^ want) <= 2, f"resumed b={b}: selection"  # at most one tie swap
        if got == want:
            check_close(to_np(out)[b, 0], ores["out"][b, 63], ATOL[dt], f"resumed b={b}",
                        kind=f"layer out {dt}")
            check_close(lse.cpu().numpy()[b, 0], ores["lse"][b, 63], LSE_ATOL[dt],
                        f"resumed b={b} lse", kind=f"layer lse {dt}")
            compared += 1
    assert compared > 0, "every row's selection was a tie swap: nothing compared"
