"""The C-ABI library: loads, exports every function include/dsa.h declares,
its struct layouts match the binding, and host-side validation returns the
documented codes without launching anything (no GPU needed)."""

import ctypes
import os
import re

import numpy as np
import pytest

from sparse_long_context_c4a_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dsa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = _declared_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_struct_layouts_match():
    for name, st in _lib.STRUCTS.items():
        assert _lib._lib.dsa_abi_sizeof(name.encode()) == ctypes.sizeof(st)
    assert _lib._lib.dsa_abi_sizeof(b"nope") == 0


def test_counts_and_version():
    assert _lib.n_complete(1048576, 4, 8) == 262143
    assert _lib.n_complete(1048576, 128, 128) == 8192
    assert _lib.n_complete(7, 4, 8) == 0 and _lib.n_complete(8, 4, 8) == 1
    assert _lib.n_complete(10, 0, 8) == -1
    assert "gfx950" in _lib.version()


def _fake(n):
    return n  # any non-zero address: validation never dereferences pointers


def _compress_args(**kw):
    a = _lib.CompressArgs()
    a.geom = _lib.geom(4, 8, 512, 64)
    a.batch, a.raw, a.raw_dtype, a.raw_len = 1, _fake(256), _lib.DSA_BF16, 16
    a.ring, a.raw_pos0, a.logits, a.logits_rows = _fake(512), _fake(768), _fake(1024), 4
    a.out, a.out_dtype, a.e_cap, a.max_pos_end = _fake(2048), _lib.DSA_BF16, 100, 400
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("raw", None), ("ring", None), ("logits_rows", 3), ("raw_dtype", 2),
    ("out_dtype", 7), ("e_cap", 0), ("max_pos_end", 8)])
def test_compress_rejects(field, value):
    with pytest.raises(_lib.DsaError) as e:
        _lib.compress(_compress_args(**{field: value}), stream=_NullStream())
    assert e.value.code == -1


def test_compress_geometry_and_fp8_scale_rejects():
    a = _compress_args()
    a.geom = _lib.geom(8, 4, 512, 64)  # span < stride
    with pytest.raises(_lib.DsaError):
        _lib.compress(a, stream=_NullStream())
    a = _compress_args(out_dtype=_lib.DSA_FP8_E4M3)  # no out_scale
    with pytest.raises(_lib.DsaError) as e:
        _lib.compress(a, stream=_NullStream())
    assert "out_scale" in str(e.value)
    a = _compress_args()
    a.geom = _lib.geom(4, 8, 512, 66)  # rope_dim > dim? no: odd pairs ok; 66 is even
    a.geom = _lib.geom(4, 8, 512, 63)  # odd rope_dim
    with pytest.raises(_lib.DsaError):
        _lib.compress(a, stream=_NullStream())


class _NullStream:
    cuda_stream = 0


def _index_args(**kw):
    a = _lib.IndexArgs()
    a.n_seqs, a.queries_per_seq, a.q_pos = 2, 1, _fake(256)
    a.stride, a.span, a.heads, a.dim = 4, 8, 16, 128
    a.q, a.q_scale, a.w, a.keys, a.k_scale = _fake(512), _fake(768), _fake(1024), _fake(2048), _fake(4096)
    a.dtype, a.e_cap, a.max_pos_end, a.k = _lib.DSA_FP8_E4M3, 1000, 4000, 64
    a.idx_out = _fake(8192)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value", [
    ("k", 0), ("q_pos", None), ("idx_out", None), ("dtype", _lib.DSA_BF16), ("k_scale", None),
    ("n_seqs", 0), ("span", 2)])
def test_index_rejects(field, value):
    a = _index_args(**{field: value})
    assert _lib.index_topk_workspace(a) == 0
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_index_topk(ctypes.byref(a), None, 0, None))
    assert e.value.code == -1


def test_index_workspace_and_null_keys():
    a = _index_args()
    need = _lib.index_topk_workspace(a)
    assert need > 0
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_index_topk(ctypes.byref(a), _fake(65536), need - 1, None))
    assert e.value.code == -3
    # keys may be NULL only when k covers every visible entry
    with pytest.raises(_lib.DsaError):
        _lib._check(_lib._lib.dsa_index_topk(ctypes.byref(_index_args(keys=None)), None, 0, None))
    ok = _index_args(keys=None, k=2000)
    assert _lib.index_topk_workspace(ok) >= 0


def _attn_args(**kw):
    a = _lib.AttnArgs()
    a.n_seqs, a.queries_per_seq, a.q_pos, a.heads, a.dim = 1, 1, _fake(256), 64, 512
    a.rope_dim, a.rope_base, a.dtype, a.q, a.rotate_q = 64, 10000.0, _lib.DSA_BF16, _fake(512), 1
    a.cache, a.e_cap, a.idx, a.k = _fake(1024), 100, _fake(2048), 64
    a.window, a.w_cap, a.window_size = _fake(4096), 128, 128
    a.max_pos_end, a.out = 400, _fake(8192)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value", [
    ("dtype", _lib.DSA_FP8_E4M3), ("w_cap", 64), ("idx", None), ("out", None), ("dim", 511),
    ("rope_dim", 600)])
def test_attn_rejects(field, value):
    a = _attn_args(**{field: value})
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_sparse_attn(ctypes.byref(a), None, 0, None))
    assert e.value.code == -1


def test_attn_unsupported_dim_and_workspace():
    a = _attn_args(dim=2048, rope_dim=64)
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_sparse_attn(ctypes.byref(a), None, 0, None))
    assert e.value.code in (-2, -3)
    a = _attn_args(n_seqs=16)
    need = _lib.sparse_attn_workspace(a)
    if need:
        with pytest.raises(_lib.DsaError) as e:
            _lib._check(_lib._lib.dsa_sparse_attn(ctypes.byref(a), None, 0, None))
        assert e.value.code == -3


def _layer_args(**kw):
    a = _lib.LayerArgs()
    a.main = _lib.geom(4, 8, 512, 64)
    a.heads, a.idx_heads, a.idx_dim, a.k, a.window_size = 64, 16, 128, 512, 128
    a.n_seqs, a.chunk_len, a.pos0, a.max_pos_end = 2, 1, _fake(256), 4096
    a.dtype, a.idx_dtype = _lib.DSA_BF16, _lib.DSA_FP8_E4M3
    for i, n in enumerate(["x", "kx", "logits_main", "logits_idx", "q", "qi", "qi_scale", "w",
                           "main_cache", "idx_cache", "idx_scale", "main_ring", "idx_ring",
                           "window", "out"]):
        setattr(a, n, _fake(4096 * (i + 1)))
    a.e_cap, a.w_cap = 1024, 128
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value", [
    ("chunk_len", 2), ("e_cap", 1023), ("w_cap", 64), ("idx_scale", None), ("kx", None),
    ("idx_dtype", _lib.DSA_BF16), ("dtype", _lib.DSA_FP8_E4M3), ("pos0", None)])
def test_layer_decode_rejects(field, value):
    a = _layer_args(**{field: value})
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_layer_decode(ctypes.byref(a), None, 0, None))
    assert e.value.code == -1


def test_layer_without_indexer_needs_k_over_n_vis():
    a = _layer_args(idx_heads=0, k=512)
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_layer_decode(ctypes.byref(a), None, 0, None))
    assert "k" in str(e.value)
    a = _layer_args(idx_heads=0, k=2000)
    need = _lib.layer_workspace(a)
    assert need > 0
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_layer_decode(ctypes.byref(a), None, 0, None))
    assert e.value.code == -3
    a = _layer_args(chunk_len=7)
    assert _lib.layer_workspace(a) > 0


@pytest.mark.parametrize("kw", [dict(k=100), dict(heads=40), dict(n_seqs=600)])
def test_layer_fp8_main_cache_shapes_refused_before_launch(kw):
    """An fp8 main cache is read by the decode attention only, which takes k
    a multiple of 32, heads a multiple of 16 and rows * heads / 16 <= 2048;
    other shapes are refused by the host checks (DSA_ERR_UNSUPPORTED) before
    the step writes any state -- here with no workspace and no GPU, so a
    launch would have failed differently."""
    a = _layer_args(main_fp8=1, main_scale=_fake(99 * 4096), **kw)
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_layer_decode(ctypes.byref(a), None, 0, None))
    assert e.value.code == -2, str(e.value)
    assert "fp8" in str(e.value)
    ok = _layer_args(main_fp8=1, main_scale=_fake(99 * 4096))
    assert _lib.layer_workspace(ok) > 0


def test_idx_tile_layout_roundtrip_and_offsets():
    """The key tile layout helpers: a byte permutation whose inverse restores
    the rows, and whose positions follow the documented offset formula."""
    import torch
    from sparse_long_context_c4a_amd.layer import idx_rows, idx_tiles
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(2, 37, 128), dtype=np.uint8)
    t = idx_tiles(codes)
    assert t.shape == (2, 48, 128)
    assert np.array_equal(idx_rows(t, 37).numpy(), codes)
    flat = t.reshape(-1).numpy()
    e_pad = 48
    for b, j, d in [(0, 0, 0), (0, 5, 17), (1, 36, 127), (1, 16, 64), (0, 31, 15)]:
        off = (b * e_pad + 16 * (j // 16)) * 128 + (d // 16) * 256 + (j % 16) * 16 + d % 16
        assert flat[off] == codes[b, j, d]


def test_layer_decode_noalloc_refuses_steps_beyond_its_scratch():
    """The allocation-free decode holds a fixed static scratch; a step whose
    workspace exceeds it is refused on the host (DSA_ERR_WORKSPACE) before
    any device call -- here without a GPU."""
    cap = _lib._lib.dsa_layer_decode_noalloc_capacity()
    assert cap == 64 << 20
    big = _layer_args(main=_lib.geom(128, 128, 512, 64), idx_heads=0, k=8192, n_seqs=256,
                      max_pos_end=1 << 20, e_cap=8192, w_cap=256)
    need = _lib.layer_workspace(big)
    assert need > cap
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_layer_decode_noalloc(ctypes.byref(big), None))
    assert e.value.code == -3 and "static scratch" in str(e.value)
    # invalid arguments are reported as by dsa_layer_decode
    bad = _layer_args(chunk_len=2)
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_layer_decode_noalloc(ctypes.byref(bad), None))
    assert e.value.code == -1


def _paging(**kw):
    p = _lib.Paging()
    p.block_table, p.swa_block_table, p.state_block = _fake(1 << 20), _fake(2 << 20), _fake(3 << 20)
    p.blocks_per_seq, p.entries_per_block = 16, 64
    p.n_blocks, p.n_swa_blocks, p.n_state_blocks = 40, 40, 3
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,code", [
    (dict(), -3),                                   # valid: only the workspace is missing
    (dict(entries_per_block=48), -1),               # not a power of two
    (dict(entries_per_block=32), -1),               # 32 * stride 4 != 256 positions
    (dict(blocks_per_seq=15), -1),                  # 15 * 64 < e_cap 1024; window < 4096
    (dict(n_blocks=0), -1),
    (dict(n_swa_blocks=0), -1),
    (dict(n_state_blocks=0), -1),
    (dict(blocks_per_seq=0), -1),
])
def test_layer_paging_validation(kw, code):
    """dsa_paging: entries_per_block a power of two equal to 256 / stride,
    the tables long enough for e_cap entries and max_pos_end positions, and
    non-empty pools; a valid paging passes (the call then asks for its
    workspace)."""
    a = _layer_args(paging=_paging(**kw), w_cap=0)
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_layer_decode(ctypes.byref(a), None, 0, None))
    assert e.value.code == code, str(e.value)


def test_paging_key_tiles_need_whole_tiles_per_block():
    """Indexer keys in 16-entry tiles cannot be paged in blocks of fewer than
    16 entries (stride 32 -> 8 entries per block): unsupported."""
    a = _index_args(stride=32, span=32, max_pos_end=4096, e_cap=128,
                    paging=_paging(entries_per_block=8, blocks_per_seq=16))
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_index_topk(ctypes.byref(a), None, 0, None))
    assert e.value.code == -2, str(e.value)
    # the same keys in f32 rows page fine (validation passes)
    a = _index_args(stride=32, span=32, max_pos_end=4096, e_cap=128, dtype=_lib.DSA_F32,
                    k_scale=None, paging=_paging(entries_per_block=8, blocks_per_seq=16))
    assert _lib.index_topk_workspace(a) > 0


def test_attention_window_table_replaces_w_cap():
    """A window table stands in for the ring (w_cap unused): without one,
    w_cap = 0 is refused."""
    a = _attn_args(w_cap=0, n_seqs=16, k=512)
    assert _lib.sparse_attn_workspace(a) == 0
    p = _paging(block_table=None, state_block=None)
    a = _attn_args(w_cap=0, n_seqs=16, k=512, paging=p)
    need = _lib.sparse_attn_workspace(a)
    assert need > 0
    with pytest.raises(_lib.DsaError) as e:
        _lib._check(_lib._lib.dsa_sparse_attn(ctypes.byref(a), None, 0, None))
    assert e.value.code == -3
