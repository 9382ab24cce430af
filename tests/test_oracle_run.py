"""Pins of the oracle's driver (oracle/run.py): the storage decoding, the
lazy row access with the rows a step writes, and run_layer itself.

Every GPU parity test builds its expected values through run_layer, which
decodes the stored bit patterns row by row (LazyRows) instead of decoding
whole caches.  These tests check it against layer_chunk run on caches that
the test decodes in full, independently of the driver (bf16 bits shifted
into binary32, fp8 codes through the e4m3fn codec times their scales), on:

* a c4a decode step over an fp8 indexer cache;
* a prefill chunk in which entries complete mid-chunk and later rows of the
  same chunk select them -- the reading that entries completing inside a
  chunk are visible to its later queries ("DeepSeek DSA、DeepSeek V4与vLLM
  Hybrid KV Cache详解" 4.1 / 4.2; "DeepSeek V4 稀疏注意力完全解剖" 机制二),
  which exercises the slice reads of rows written by the step;
* a decode step over a token-wise fp8 main cache (codes times one scale per
  entry);
* a c128a decode step, which has no indexer;
* a decode step over an MXFP4 indexer cache (E2M1 codes from a magnitude
  table written here, times 2^(scale byte - 127) per 32 dims), with fp8
  indexer queries.

The outputs, selections and final states must be equal element by element:
both sides run the same float64 arithmetic on the same values, so any
difference is a decoding or override mistake in the driver.
"""

import numpy as np
import pytest

from oracle import codecs, dsa
from oracle.layer import Geometry, SeqState, layer_chunk
from oracle.run import LazyRows, decode_store, run_layer
from sparse_long_context_c4a_amd import configs, inputs as gen


def _bf16(bits):
    # bf16 is the high half of a binary32 pattern
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _full(bits, dtype, scale=None):
    if bits is None:
        return None
    if dtype == "f32":
        return np.asarray(bits, np.float32).astype(np.float64)
    if dtype == "bf16":
        return _bf16(bits)
    if dtype == "fp4":
        # E2M1 magnitudes by code (OCP MX FP4), bit 3 the sign; one E8M0
        # scale byte per 32 dims
        mag = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
        c = np.asarray(bits, np.int64)
        v = mag[c & 7] * (1.0 - 2.0 * ((c >> 3) & 1))
        x = 2.0 ** (np.asarray(scale, np.float64) - 127.0)
        return v * np.repeat(x, 32, axis=-1)
    assert dtype == "fp8"
    return codecs.fp8_decode(bits) * np.asarray(scale, np.float64)[..., None]


def _geom(w):
    return Geometry(s=w.s, S=w.S, D=w.D, r=w.r, Di=w.Di, r_idx=w.r_idx, H=w.H, Hi=w.Hi, k=w.k,
                    W=w.W, base=w.base, base_idx=w.base, main_dtype=w.main_dtype,
                    idx_dtype=w.idx_dtype, main_cache_dtype=w.main_cache_dtype)


def _reference(w, inp):
    """layer_chunk per sequence on fully decoded float64 state arrays."""
    g = _geom(w)
    B, T = inp["x"].shape[0], inp["T"]
    mcd = w.main_cache_dtype or w.main_dtype
    rdt = "f32" if w.idx_dtype == "f32" else "bf16"
    res = dict(out=np.zeros((B, T, w.H, w.D)), lse=np.zeros((B, T, w.H)),
               idx=np.full((B, T, w.k), -1, np.int64), states=[])
    for b in range(B):
        msc = None if inp["main_scale"] is None else inp["main_scale"][b]
        main = _full(inp["main_cache"][b], mcd, msc)
        if w.Hi:
            if w.idx_dtype == "fp4":
                isc = inp["idx_mx"][b]
            else:
                isc = None if inp["idx_scale"] is None else inp["idx_scale"][b]
            idxc = _full(inp["idx_cache"][b], w.idx_dtype, isc)
            iring = _full(inp["idx_ring"][b], rdt)
            kx = _full(inp["kx"][b], rdt)
            qsc = None if inp["qi_scale"] is None else inp["qi_scale"][b]
            qi = _full(inp["qi"][b], "fp8" if w.idx_dtype == "fp4" else w.idx_dtype, qsc)
            wt = np.asarray(inp["wt"][b], np.float64)
            lgi = np.asarray(inp["logits_idx"][b], np.float64)
        else:
            idxc = np.zeros((inp["E_cap"], 0))
            iring = np.zeros((w.S, 0))
            kx = np.zeros((T, 0))
            qi = np.zeros((T, 0, 0))
            wt = np.zeros((T, 0))
            lgi = np.zeros((inp["n_new"], w.S))
        st = SeqState(main_cache=main, idx_cache=idxc, idx_scale=np.ones(inp["E_cap"]),
                      main_ring=_full(inp["main_ring"][b], w.main_dtype), idx_ring=iring,
                      win_ring=_full(inp["win_ring"][b], w.main_dtype))
        o, l, ix = layer_chunk(g, st, inp["p0"], _full(inp["x"][b], w.main_dtype), kx,
                               np.asarray(inp["logits_main"][b], np.float64), lgi,
                               _full(inp["q"][b], w.main_dtype), qi, wt)
        res["out"][b], res["lse"][b], res["idx"][b] = o, l, ix
        res["states"].append(st)
    return res


def _rows(c, n):
    return np.stack([c[j] for j in range(n)])


def _assert_same(w, inp, got, ref):
    assert np.array_equal(got["idx"], ref["idx"])
    assert np.array_equal(got["out"], ref["out"])
    assert np.array_equal(got["lse"], ref["lse"])
    E = inp["E_cap"]
    for sg, sr in zip(got["states"], ref["states"]):
        assert np.array_equal(_rows(sg.main_cache, E), sr.main_cache)
        if w.Hi:
            assert np.array_equal(_rows(sg.idx_cache, E), sr.idx_cache)
        assert np.array_equal(sg.main_ring, sr.main_ring)
        assert np.array_equal(sg.idx_ring, sr.idx_ring)
        assert np.array_equal(sg.win_ring, sr.win_ring)


CASES = [
    # name, workload, overrides, p0, T
    ("c4a_decode_fp8_index", configs.C4A_DECODE_64K, dict(B=2, L=3000, H=8), None, None),
    ("c4a_prefill_mid_chunk_entries", configs.C4A_PREFILL_128K,
     dict(L=364, k=24, H=8), 300, 64),
    ("c4a_decode_fp8_main_cache", configs.C4A_DECODE_64K,
     dict(B=2, L=2000, H=8, main_cache_dtype="fp8"), None, None),
    ("c128a_decode_no_indexer", configs.C128A_DECODE_1M, dict(B=2, L=5120, k=64, H=8), None,
     None),
    ("c4a_decode_fp4_index", configs.C4A_DECODE_1M_FP4, dict(B=2, L=3000, H=8), None, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_run_layer_equals_layer_chunk_on_decoded_state(case):
    name, w0, over, p0, T = case
    w = configs.shrink(w0, **over)
    inp = gen.layer_inputs(w, seed=9100 + CASES.index(case), p0=p0, T=T, state="random")
    got = run_layer(_geom(w), inp)
    ref = _reference(w, inp)
    _assert_same(w, inp, got, ref)
    if name == "c4a_prefill_mid_chunk_entries":
        # the chunk completes entries j0 .. j0+n_new-1; later rows must both
        # see and select some of them, or the slice reads were not exercised
        j0, n_new = inp["j0"], inp["n_new"]
        assert n_new >= 10
        sel_new = (got["idx"] >= j0) & (got["idx"] < j0 + n_new)
        assert sel_new.sum() >= 10, sel_new.sum()
        # and the written rows differ from the random bits the slots held
        assert not np.array_equal(_rows(got["states"][0].main_cache, j0 + n_new)[j0:],
                                  _full(inp["main_cache"][0][j0:j0 + n_new], "bf16"))
    if name == "c128a_decode_no_indexer":
        m = inp["p0"]
        nv = dsa.n_vis(m, w.s, w.S)
        assert sorted(got["idx"][0, 0][got["idx"][0, 0] >= 0].tolist()) == list(range(nv))


def test_decode_store_fp8_is_code_value_times_scale():
    # e4m3fn values written out: 0x38 = 1.0, 0x40 = 2.0, 0xB8 = -1.0,
    # 0x7E = 448 (largest finite), 0x01 = 2^-9 (smallest subnormal),
    # 0x08 = 2^-6 (smallest normal), 0x3C = 1.5, 0x00 = 0
    codes = np.array([[0x38, 0x40, 0xB8, 0x7E], [0x01, 0x08, 0x3C, 0x00]], np.uint8)
    scale = np.array([0.5, 3.0], np.float32)
    want = np.array([[0.5, 1.0, -0.5, 224.0], [3.0 * 2.0 ** -9, 3.0 * 2.0 ** -6, 4.5, 0.0]])
    assert np.array_equal(decode_store(codes, "fp8", scale), want)
    # bf16 bits: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25, 0x7F7F = largest finite
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x7F7F], np.uint16)
    assert np.array_equal(decode_store(bits, "bf16"),
                          np.array([1.0, -2.0, 0.25, (2.0 - 2.0 ** -7) * 2.0 ** 127]))
    f = np.array([1.5, -0.1], np.float32)
    assert np.array_equal(decode_store(f, "f32"), f.astype(np.float64))
    assert decode_store(None, "bf16") is None


def test_lazy_rows_slices_apply_written_rows():
    rng = np.random.default_rng(3)
    codes = gen.to_fp8_codes(rng.standard_normal((10, 4)) * 64)
    scale = np.linspace(0.5, 1.4, 10).astype(np.float32)
    lz = LazyRows(codes, "fp8", scale)
    full = codecs.fp8_decode(codes) * scale.astype(np.float64)[:, None]
    assert np.array_equal(lz[2:7], full[2:7])
    assert np.array_equal(lz[4], full[4])
    v6, v9 = np.full(4, 6.25), np.full(4, -9.5)
    lz[6] = v6
    lz[9] = v9
    exp = full.copy()
    exp[6], exp[9] = v6, v9
    assert np.array_equal(lz[:10], exp)
    assert np.array_equal(lz[5:8], exp[5:8])
    assert np.array_equal(lz[0:10:3], exp[0:10:3])   # rows 0, 3, 6, 9: both overrides
    assert np.array_equal(lz[1:10:4], exp[1:10:4])   # rows 1, 5, 9
    assert np.array_equal(lz[:6], exp[:6])            # row 6 outside the slice
    assert np.array_equal(lz[6], v6)
