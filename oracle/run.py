"""Drive the oracle from a dict of stored inputs (bit patterns).

Test infrastructure only (see the package docstring).  Decodes the storage
formats with ``oracle.codecs`` and runs ``oracle.layer.layer_chunk`` per
sequence.  Large caches are decoded lazily, row by row, so that a 1M-token
context does not need a float64 copy of the whole main cache.
"""

import numpy as np

from . import codecs
from . import dsa
from .layer import Geometry, SeqState, layer_chunk


def decode_store(a, dtype, scale=None):
    """Stored array -> float64 values (fp8 rows times their scales)."""
    if a is None:
        return None
    if dtype == "f64":
        return np.asarray(a, np.float64)
    if dtype == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    if dtype == "bf16":
        return codecs.bf16_decode(a)
    if dtype == "fp8":
        v = codecs.fp8_decode(a)
        return v * np.asarray(scale, np.float64)[..., None]
    if dtype == "fp4":  # MXFP4 codes with their E8M0 block scales
        return dsa.mxfp4_decode(a, scale)
    raise ValueError(dtype)


class LazyRows:
    """Row access into a stored [E, D] array, decoding on demand; rows that
    the layer writes are kept as float64 overrides."""

    def __init__(self, bits, dtype, scale=None):
        self.bits, self.dtype, self.scale = bits, dtype, scale
        self.over = {}
        self.shape = bits.shape

    def __getitem__(self, key):
        if isinstance(key, slice):
            start, stop, step = key.indices(self.shape[0])
            rows = decode_store(self.bits[start:stop:step], self.dtype,
                                None if self.scale is None else self.scale[start:stop:step])
            for j, v in self.over.items():
                if start <= j < stop and (j - start) % step == 0:
                    rows[(j - start) // step] = v
            return rows
        j = int(key)
        if j in self.over:
            return self.over[j]
        return decode_store(self.bits[j], self.dtype,
                            None if self.scale is None else self.scale[j])

    def __setitem__(self, j, v):
        self.over[int(j)] = np.asarray(v, np.float64)


class _Unit:
    """Stand-in indexer cache for layers without an indexer."""

    def __getitem__(self, key):
        return np.zeros((0, 0))

    def __setitem__(self, j, v):
        pass


def raw_dtype_idx(idx_dtype):
    return "f32" if idx_dtype == "f32" else "bf16"


def q_dtype_idx(idx_dtype):
    """The indexer queries' storage: fp8 beside fp4 keys, else the keys'."""
    return "fp8" if idx_dtype == "fp4" else idx_dtype


def run_layer(g: Geometry, inp, only=None, rotate_q=True, alt_idx=None):
    """Run one layer step for every sequence of ``inp`` (the dict produced by
    the seeded generator).  ``only``: optional list of chunk offsets t whose
    outputs are wanted (others are skipped; the state update is complete).
    ``alt_idx`` [B, T, k] (optional): per-row selections to also attend over
    where they differ from the oracle's (see ``layer_chunk``).

    Returns dict(out [B, T, H, D], lse [B, T, H], idx [B, T, k],
    states [per-sequence SeqState]).
    """
    B = inp["x"].shape[0]
    T = inp["T"]
    p0 = inp["p0"]
    has_idx = g.Hi > 0
    rdt = raw_dtype_idx(g.idx_dtype)
    outs = np.zeros((B, T, g.H, g.D))
    lses = np.zeros((B, T, g.H))
    idxs = np.full((B, T, g.k), -1, np.int64)
    states = []
    for b in range(B):
        msc = inp.get("main_scale")
        main = LazyRows(inp["main_cache"][b], g.main_cache_dtype or g.main_dtype,
                        None if msc is None else msc[b])
        if has_idx:
            if g.idx_dtype == "fp4":
                sc = inp["idx_mx"][b]
            else:
                sc = None if inp["idx_scale"] is None else inp["idx_scale"][b]
            idxc = LazyRows(inp["idx_cache"][b], g.idx_dtype, sc)
            idx_ring = decode_store(inp["idx_ring"][b], rdt)
            kx = decode_store(inp["kx"][b], rdt)
            qi = decode_store(inp["qi"][b], q_dtype_idx(g.idx_dtype),
                              None if inp["qi_scale"] is None else inp["qi_scale"][b])
            wt = np.asarray(inp["wt"][b], np.float64)
            lg_idx = np.asarray(inp["logits_idx"][b], np.float64)
        else:
            idxc = _Unit()
            idx_ring = np.zeros((g.S, 0))
            kx = np.zeros((T, 0))
            qi = np.zeros((T, 0, 0))
            wt = np.zeros((T, 0))
            lg_idx = np.zeros((inp["n_new"], g.S))
        st = SeqState(main_cache=main, idx_cache=idxc,
                      idx_scale=np.ones(inp["E_cap"]),
                      main_ring=decode_store(inp["main_ring"][b], g.main_dtype),
                      idx_ring=idx_ring,
                      win_ring=decode_store(inp["win_ring"][b], g.main_dtype))
        x = decode_store(inp["x"][b], g.main_dtype)
        q = decode_store(inp["q"][b], g.main_dtype)
        o, l, ix = layer_chunk(g, st, p0, x, kx,
                               np.asarray(inp["logits_main"][b], np.float64), lg_idx,
                               q, qi, wt, rotate_q=rotate_q, only=only,
                               alt_idx=None if alt_idx is None else alt_idx[b])
        outs[b], lses[b], idxs[b] = o, l, ix
        states.append(st)
    return dict(out=outs, lse=lses, idx=idxs, states=states)
