"""Marshalling for one layer step: torch tensors in, LayerArgs out.

Holds no arithmetic of the layer; it moves the seeded inputs to the device,
keeps the state tensors (caches, compressor rings, window ring) and fills
the C structs of the library.
"""

from dataclasses import dataclass

import numpy as np
import torch

from . import _lib
from .configs import Workload


def to_device(a, device="cuda"):
    """NumPy storage array -> device tensor with the same bits (uint16 bf16
    patterns become torch.bfloat16, fp8 codes stay uint8)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def idx_tiles(codes):
    """fp8 key codes [B, E, 128] (NumPy uint8 or tensor) -> the library's
    16-entry tile layout [B, E_pad, 128] (E_pad = E rounded up to 16): each
    tile of 16 entries is stored chunk-major (8 chunks of 16 bytes, each the
    16 entries' bytes of that chunk).  A pure permutation of bytes."""
    t = codes if isinstance(codes, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(codes))
    B, E, D = t.shape
    assert D == 128
    Ep = -(-E // 16) * 16
    if Ep != E:
        t = torch.cat([t, torch.zeros((B, Ep - E, D), dtype=t.dtype, device=t.device)], dim=1)
    return t.reshape(B, Ep // 16, 16, 8, 16).permute(0, 1, 3, 2, 4).contiguous().reshape(B, Ep, D)


def idx_rows(tiles, E):
    """Inverse of idx_tiles: [B, E_pad, 128] tile layout -> [B, E, 128]."""
    B, Ep, D = tiles.shape
    t = tiles.reshape(B, Ep // 16, 8, 16, 16).permute(0, 1, 3, 2, 4).contiguous()
    return t.reshape(B, Ep, D)[:, :E]


def idx4_tiles(codes):
    """fp4 key codes [B, E, 128] (one E2M1 code 0..15 per byte) -> the
    library's fp4 tile layout [B, E_pad, 64]: two codes per byte (the even
    dim in the lower nibble), each 16-entry tile stored chunk-major (4 chunks
    of 32 dims = 16 bytes, each the 16 entries' bytes of that chunk)."""
    t = codes if isinstance(codes, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(codes))
    B, E, D = t.shape
    assert D == 128
    packed = (t[..., 0::2] & 15) | ((t[..., 1::2] & 15) << 4)
    Ep = -(-E // 16) * 16
    if Ep != E:
        packed = torch.cat([packed, torch.zeros((B, Ep - E, 64), dtype=packed.dtype,
                                                device=packed.device)], dim=1)
    return packed.reshape(B, Ep // 16, 16, 4, 16).permute(0, 1, 3, 2, 4).contiguous().reshape(B, Ep, 64)


def idx4_rows(tiles, E):
    """Inverse of idx4_tiles: [B, E_pad, 64] fp4 tiles -> codes [B, E, 128]."""
    B, Ep, _ = tiles.shape
    t = tiles.reshape(B, Ep // 16, 4, 16, 16).permute(0, 1, 3, 2, 4).contiguous()
    t = t.reshape(B, Ep, 64)[:, :E]
    out = torch.empty((B, E, 128), dtype=t.dtype, device=t.device)
    out[..., 0::2] = t & 15
    out[..., 1::2] = t >> 4
    return out


def idx_to_device(codes, device="cuda", fp4=False):
    """Indexer keys to the device: fp8 (or, with fp4, E2M1) codes of dim 128
    in the tile layout, anything else (f32, other dims) unchanged."""
    if codes is None:
        return None
    if codes.dtype == np.uint8 and codes.ndim == 3 and codes.shape[-1] == 128:
        return (idx4_tiles(codes) if fp4 else idx_tiles(codes)).to(device)
    return to_device(codes, device)


@dataclass
class LayerState:
    main_cache: torch.Tensor
    idx_cache: torch.Tensor
    idx_scale: torch.Tensor
    main_ring: torch.Tensor
    idx_ring: torch.Tensor
    window: torch.Tensor
    e_cap: int
    main_scale: torch.Tensor = None  # token-wise fp8 main cache: one scale per entry
    idx_mx: torch.Tensor = None      # fp4 indexer cache: E8M0 scale bytes [B, e_cap, Di / 32]


@dataclass
class Chunk:
    pos0: torch.Tensor      # [B] int64
    T: int
    x: torch.Tensor
    kx: torch.Tensor
    logits_main: torch.Tensor
    logits_idx: torch.Tensor
    q: torch.Tensor
    qi: torch.Tensor
    qi_scale: torch.Tensor
    w: torch.Tensor


def state_from_inputs(inp, device="cuda"):
    mx = inp.get("idx_mx")
    return LayerState(main_cache=to_device(inp["main_cache"], device),
                      idx_cache=idx_to_device(inp["idx_cache"], device, fp4=mx is not None),
                      idx_scale=to_device(inp["idx_scale"], device),
                      main_ring=to_device(inp["main_ring"], device),
                      idx_ring=to_device(inp["idx_ring"], device),
                      window=to_device(inp["win_ring"], device),
                      e_cap=int(inp["E_cap"]),
                      main_scale=to_device(inp.get("main_scale"), device),
                      idx_mx=to_device(mx, device))


def _pad_logits(lg, rows):
    if lg is None:
        return None
    B, n, S = lg.shape
    out = np.zeros((B, max(rows, 1), S), np.float32)
    out[:, :n] = lg
    return out


def chunk_from_inputs(w: Workload, inp, device="cuda"):
    B, T = inp["x"].shape[0], inp["T"]
    rows = -(-T // w.s)
    return Chunk(pos0=torch.full((B,), inp["p0"], dtype=torch.int64, device=device), T=T,
                 x=to_device(inp["x"], device), kx=to_device(inp["kx"], device),
                 logits_main=to_device(_pad_logits(inp["logits_main"], rows), device),
                 logits_idx=to_device(_pad_logits(inp["logits_idx"], rows), device),
                 q=to_device(inp["q"], device), qi=to_device(inp["qi"], device),
                 qi_scale=to_device(inp["qi_scale"], device), w=to_device(inp["wt"], device))


def layer_args(w: Workload, st: LayerState, ch: Chunk, out, lse=None, idx_out=None,
               status=None, max_pos_end=None, pos_offset=0, rms_gamma=None,
               rms_gamma_idx=None, rms_eps=1e-6, softmax_scale=0.0, out_scale=None,
               q_norm_gamma=None, pages=None):
    a = _lib.LayerArgs()
    a.main = _lib.geom(w.s, w.S, w.D, w.r, w.base, pos_offset)
    a.heads, a.idx_heads, a.idx_dim = w.H, w.Hi, w.Di
    a.idx_rope_dim, a.idx_rope_base = w.r_idx, w.base
    a.k, a.window_size, a.softmax_scale = w.k, w.W, softmax_scale
    a.n_seqs, a.chunk_len = ch.x.shape[0], ch.T
    a.pos0 = _lib.ptr(ch.pos0)
    a.max_pos_end = max_pos_end if max_pos_end is not None else st.e_cap * w.s
    a.dtype = _lib.DSA_F32 if w.main_dtype == "f32" else _lib.DSA_BF16
    a.idx_dtype = {"f32": _lib.DSA_F32, "fp8": _lib.DSA_FP8_E4M3,
                   "fp4": _lib.DSA_FP4_E2M1}[w.idx_dtype]
    for name in ("x", "kx", "logits_main", "logits_idx", "q", "qi", "qi_scale", "w"):
        setattr(a, name, _lib.ptr(getattr(ch, name)))
    a.main_cache, a.idx_cache = _lib.ptr(st.main_cache), _lib.ptr(st.idx_cache)
    a.idx_scale, a.e_cap = _lib.ptr(st.idx_scale), st.e_cap
    a.idx_mx_scale = _lib.ptr(st.idx_mx)
    a.main_ring, a.idx_ring = _lib.ptr(st.main_ring), _lib.ptr(st.idx_ring)
    a.window, a.w_cap = _lib.ptr(st.window), st.window.shape[1]
    if pages is not None:  # block tables; the state's tensors are the pools
        a.paging = pages.args()
        a.w_cap = 0
    a.rms_gamma, a.rms_gamma_idx, a.rms_eps = _lib.ptr(rms_gamma), _lib.ptr(rms_gamma_idx), rms_eps
    a.q_norm_gamma = _lib.ptr(q_norm_gamma)
    if st.main_scale is not None:  # fp8 codes in main_cache
        a.main_fp8, a.main_scale = 1, _lib.ptr(st.main_scale)
    a.out, a.lse, a.idx_out = _lib.ptr(out), _lib.ptr(lse), _lib.ptr(idx_out)
    if out_scale is not None:  # fp8 output codes in out, one scale per (b, t, head)
        a.out_fp8, a.out_scale = 1, _lib.ptr(out_scale)
    a.status = _lib.ptr(status)
    return a


def alloc_outputs(w: Workload, B, T, device="cuda", out_fp8=False):
    dt = torch.float32 if w.main_dtype == "f32" else torch.bfloat16
    if out_fp8:
        dt = torch.uint8
    out = torch.empty((B, T, w.H, w.D), dtype=dt, device=device)
    lse = torch.empty((B, T, w.H), dtype=torch.float32, device=device)
    idx = torch.empty((B, T, w.k), dtype=torch.int32, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    return out, lse, idx, status


def run(w: Workload, st: LayerState, ch: Chunk, decode=None, ws=None, out_fp8=False, **kw):
    """One layer step; returns (out, lse, idx, status, workspace).  With
    out_fp8 the output is stored as fp8 codes and out is (codes, scales)."""
    B, T = ch.x.shape[0], ch.T
    out, lse, idx, status = alloc_outputs(w, B, T, ch.x.device, out_fp8)
    osc = torch.empty((B, T, w.H), dtype=torch.float32, device=ch.x.device) if out_fp8 else None
    a = layer_args(w, st, ch, out, lse, idx, status, out_scale=osc, **kw)
    if decode is None:
        decode = T == 1
    fn = _lib.layer_decode if decode else _lib.layer_prefill
    ws = fn(a, ws=ws, device=ch.x.device)
    return (out, osc) if out_fp8 else out, lse, idx, status, ws


# ------------------------------------------------------------ paged state
@dataclass
class Pages:
    """Block tables of a paged layer state (logical block = 256 raw
    positions): entry pools hold epb = 256 / s entries per block, the window
    pool 256 tokens per block, the ring pools one sequence's rings per block."""
    table: torch.Tensor      # [B, blocks_per_seq] int32
    swa_table: torch.Tensor  # [B, blocks_per_seq] int32
    state: torch.Tensor      # [B] int32
    epb: int
    n_blocks: int
    n_swa: int
    n_state: int

    def args(self):
        p = _lib.Paging()
        p.block_table, p.swa_block_table = _lib.ptr(self.table), _lib.ptr(self.swa_table)
        p.state_block = _lib.ptr(self.state)
        p.blocks_per_seq, p.entries_per_block = self.table.shape[1], self.epb
        p.n_blocks, p.n_swa_blocks, p.n_state_blocks = self.n_blocks, self.n_swa, self.n_state
        return p


def _perm_table(gen, B, nb, n_pool):
    """Distinct physical blocks for every (sequence, logical block), drawn
    as a random permutation of a pool with spare blocks."""
    perm = torch.randperm(n_pool, generator=gen)[:B * nb]
    return perm.reshape(B, nb).to(torch.int32)


def page_state(w: Workload, st: LayerState, p0, seed=0, spare=3):
    """A paged copy of a dense state (same values, scattered over block
    pools in a seeded random order) and its block tables.  Only the window
    tokens before p0 that the ring holds are carried over."""
    dev = st.main_cache.device
    gen = torch.Generator().manual_seed(seed)
    B = st.main_cache.shape[0]
    epb = 256 // w.s
    nb = -(-st.e_cap // epb)
    nb_w = -(-(st.e_cap * w.s) // 256)
    nbps = max(nb, nb_w)
    n_blocks, n_swa, n_state = B * nbps + spare, B * nbps + spare, B + spare
    table = _perm_table(gen, B, nbps, n_blocks)
    swa = _perm_table(gen, B, nbps, n_swa)
    state = torch.randperm(n_state, generator=gen)[:B].to(torch.int32)
    rows = table.long()[:, :, None] * epb + torch.arange(epb)[None, None, :]  # [B, nbps, epb]
    rows = rows.reshape(B, nbps * epb)[:, :st.e_cap].to(dev)                 # pool row of (b, j)

    def scatter_rows(dense, per_row_shape, dtype):
        pool = torch.zeros((n_blocks * epb,) + per_row_shape, dtype=dtype, device=dev)
        if dense is not None:
            pool[rows.reshape(-1)] = dense[:, :st.e_cap].reshape((-1,) + per_row_shape)
        return pool

    def scatter_tiles(tiles, bpe):
        # dense tile layout [B, E_pad, bpe]: a block of epb entries is a
        # contiguous run of epb * bpe bytes in both layouts
        Ep = tiles.shape[1]
        pad = nbps * epb - Ep
        t = torch.cat([tiles, torch.zeros((B, pad, bpe), dtype=tiles.dtype, device=dev)], 1) \
            if pad > 0 else tiles[:, :nbps * epb]
        pool = torch.zeros((n_blocks, epb, bpe), dtype=tiles.dtype, device=dev)
        pool[table.long().reshape(-1).to(dev)] = t.reshape(B * nbps, epb, bpe)
        return pool.reshape(n_blocks * epb, bpe)

    D = st.main_cache.shape[-1]
    main = scatter_rows(st.main_cache, (D,), st.main_cache.dtype)
    main_scale = scatter_rows(st.main_scale, (), torch.float32) if st.main_scale is not None else None
    idx_cache = idx_scale = idx_mx = None
    if st.idx_cache is not None:
        if st.idx_cache.dtype == torch.uint8 and st.idx_cache.shape[-1] in (64, 128) and \
                w.Di == 128:
            idx_cache = scatter_tiles(st.idx_cache, st.idx_cache.shape[-1])
        else:
            idx_cache = scatter_rows(st.idx_cache, tuple(st.idx_cache.shape[2:]), st.idx_cache.dtype)
        if st.idx_scale is not None:
            idx_scale = scatter_rows(st.idx_scale, (), torch.float32)
        if st.idx_mx is not None:
            idx_mx = scatter_rows(st.idx_mx, (st.idx_mx.shape[-1],), torch.uint8)
    # window: tokens n in [max(0, p0 - w_cap), p0) from ring slot n mod w_cap
    w_cap = st.window.shape[1]
    win = torch.zeros((n_swa * 256, D), dtype=st.window.dtype, device=dev)
    n = torch.arange(max(0, p0 - w_cap), p0)
    if len(n):
        srow = swa.long()[:, n // 256] * 256 + (n % 256)[None, :]            # [B, len]
        win[srow.reshape(-1).to(dev)] = st.window[:, n % w_cap].reshape(-1, D)
    # rings: one block per sequence
    def scatter_state(ring):
        if ring is None:
            return None
        pool = torch.zeros((n_state,) + tuple(ring.shape[1:]), dtype=ring.dtype, device=dev)
        pool[state.long().to(dev)] = ring
        return pool
    pst = LayerState(main_cache=main, idx_cache=idx_cache, idx_scale=idx_scale,
                     main_ring=scatter_state(st.main_ring), idx_ring=scatter_state(st.idx_ring),
                     window=win.reshape(n_swa, 256, D), e_cap=st.e_cap, main_scale=main_scale,
                     idx_mx=idx_mx)
    pages = Pages(table=table.to(dev), swa_table=swa.to(dev), state=state.to(dev), epb=epb,
                  n_blocks=n_blocks, n_swa=n_swa, n_state=n_state)
    return pst, pages


def unpage_state(w: Workload, pst: LayerState, pages: Pages, like: LayerState):
    """The dense view of a paged state (caches and rings; the window as the
    tokens of positions [lo, hi) is separate: unpage_window)."""
    B = like.main_cache.shape[0]
    epb, e_cap = pages.epb, like.e_cap
    nbps = pages.table.shape[1]
    rows = (pages.table.long()[:, :, None] * epb +
            torch.arange(epb, device=pages.table.device)[None, None, :]).reshape(B, -1)[:, :e_cap]
    out = {}
    out["main_cache"] = pst.main_cache[rows]
    if pst.main_scale is not None:
        out["main_scale"] = pst.main_scale[rows]
    if pst.idx_cache is not None:
        if like.idx_cache.dtype == torch.uint8 and w.Di == 128:
            bpe = pst.idx_cache.shape[-1]
            blocks = pst.idx_cache.reshape(pages.n_blocks, epb, bpe)[pages.table.long()]
            Ep = like.idx_cache.shape[1]
            out["idx_cache"] = blocks.reshape(B, nbps * epb, bpe)[:, :Ep]
        else:
            out["idx_cache"] = pst.idx_cache[rows]
        if pst.idx_scale is not None:
            out["idx_scale"] = pst.idx_scale[rows]
        if pst.idx_mx is not None:
            out["idx_mx"] = pst.idx_mx[rows]
    out["main_ring"] = pst.main_ring[pages.state.long()]
    if pst.idx_ring is not None:
        out["idx_ring"] = pst.idx_ring[pages.state.long()]
    return out


def unpage_window(pst: LayerState, pages: Pages, lo, hi):
    """Window tokens of positions lo .. hi-1 of every sequence [B, hi-lo, D]."""
    n = torch.arange(lo, hi, device=pages.swa_table.device)
    r = pages.swa_table.long()[:, n // 256] * 256 + (n % 256)[None, :]
    D = pst.window.shape[-1]
    return pst.window.reshape(-1, D)[r]


def dense_window(st: LayerState, lo, hi):
    n = torch.arange(lo, hi, device=st.window.device)
    return st.window[:, n % st.window.shape[1]]
