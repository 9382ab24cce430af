"""ctypes binding of libdsa.so (include/dsa.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Tensors are torch tensors on the GPU (their data_ptr() is passed through);
workspace buffers are allocated here with torch and handed to the library.
There is no fallback: if the library is missing, importing this module
raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSA_LIB_PATH selects another build of the same library (same ABI)
LIB_PATH = os.environ.get("DSA_LIB_PATH") or os.path.join(_HERE, "libdsa.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3, DSA_FP4_E2M1 = 0, 1, 2, 3
STATUS = {0: "DSA_OK", -1: "DSA_ERR_INVALID_ARG", -2: "DSA_ERR_UNSUPPORTED",
          -3: "DSA_ERR_WORKSPACE", -4: "DSA_ERR_HIP"}
DEVERR_POSITION, DEVERR_CAPACITY, DEVERR_NO_INDEX, DEVERR_BLOCK = 1, 2, 4, 8
BLOCK_TOKENS = 256  # raw positions per logical block of the paged caches

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m sparse_long_context_c4a_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

c_i32, c_i64, c_f32, c_f64, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                    ctypes.c_double, ctypes.c_void_p)


class TimingEvents(ctypes.Structure):
    _fields_ = [("index_begin", c_vp), ("index_end", c_vp), ("attn_begin", c_vp),
                ("attn_end", c_vp)]


class Geom(ctypes.Structure):
    _fields_ = [("stride", c_i32), ("span", c_i32), ("dim", c_i32), ("rope_dim", c_i32),
                ("rope_base", c_f64), ("rope_pos_offset", c_i64)]


class Paging(ctypes.Structure):
    _fields_ = [("block_table", c_vp), ("swa_block_table", c_vp), ("state_block", c_vp),
                ("blocks_per_seq", c_i32), ("entries_per_block", c_i32), ("n_blocks", c_i32),
                ("n_swa_blocks", c_i32), ("n_state_blocks", c_i32)]


class CompressArgs(ctypes.Structure):
    _fields_ = [("geom", Geom), ("batch", c_i32), ("raw", c_vp), ("raw_dtype", c_i32),
                ("raw_len", c_i64), ("ring", c_vp), ("raw_pos0", c_vp), ("logits", c_vp),
                ("logits_rows", c_i32), ("rms_gamma", c_vp), ("rms_eps", c_f32), ("out", c_vp),
                ("out_dtype", c_i32), ("out_scale", c_vp), ("e_cap", c_i64),
                ("max_pos_end", c_i64), ("status", c_vp), ("out_mx_scale", c_vp),
                ("paging", Paging)]


class IndexArgs(ctypes.Structure):
    _fields_ = [("n_seqs", c_i32), ("queries_per_seq", c_i32), ("q_pos", c_vp),
                ("stride", c_i32), ("span", c_i32), ("heads", c_i32), ("dim", c_i32),
                ("q", c_vp), ("q_scale", c_vp), ("w", c_vp), ("keys", c_vp), ("k_scale", c_vp),
                ("dtype", c_i32), ("e_cap", c_i64), ("max_pos_end", c_i64), ("k", c_i32),
                ("idx_out", c_vp), ("score_out", c_vp), ("status", c_vp),
                ("k_mx_scale", c_vp), ("paging", Paging)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("n_seqs", c_i32), ("queries_per_seq", c_i32), ("q_pos", c_vp),
                ("heads", c_i32), ("dim", c_i32), ("rope_dim", c_i32), ("rope_base", c_f64),
                ("rope_pos_offset", c_i64), ("dtype", c_i32), ("q", c_vp), ("rotate_q", c_i32),
                ("cache", c_vp), ("e_cap", c_i64), ("idx", c_vp), ("k", c_i32),
                ("window", c_vp), ("w_cap", c_i32), ("window_size", c_i32),
                ("chunk_win", c_vp), ("chunk_pos0", c_vp), ("chunk_len", c_i64),
                ("softmax_scale", c_f32), ("max_pos_end", c_i64), ("out", c_vp),
                ("lse", c_vp), ("status", c_vp), ("out_fp8", c_i32), ("out_scale", c_vp),
                ("cache_fp8", c_i32), ("cache_scale", c_vp), ("paging", Paging)]


class LayerArgs(ctypes.Structure):
    _fields_ = [("main", Geom), ("heads", c_i32), ("idx_heads", c_i32), ("idx_dim", c_i32),
                ("idx_rope_dim", c_i32), ("idx_rope_base", c_f64), ("k", c_i32),
                ("window_size", c_i32), ("softmax_scale", c_f32), ("n_seqs", c_i32),
                ("chunk_len", c_i32), ("pos0", c_vp), ("max_pos_end", c_i64),
                ("dtype", c_i32), ("idx_dtype", c_i32), ("x", c_vp), ("kx", c_vp),
                ("logits_main", c_vp), ("logits_idx", c_vp), ("q", c_vp), ("qi", c_vp),
                ("qi_scale", c_vp), ("w", c_vp), ("main_cache", c_vp), ("idx_cache", c_vp),
                ("idx_scale", c_vp), ("e_cap", c_i64), ("main_ring", c_vp), ("idx_ring", c_vp),
                ("window", c_vp), ("w_cap", c_i32), ("rms_gamma", c_vp), ("rms_gamma_idx", c_vp),
                ("rms_eps", c_f32), ("out", c_vp), ("lse", c_vp), ("idx_out", c_vp),
                ("status", c_vp), ("out_fp8", c_i32), ("out_scale", c_vp), ("main_fp8", c_i32),
                ("main_scale", c_vp), ("q_norm_gamma", c_vp), ("idx_mx_scale", c_vp),
                ("paging", Paging)]


EXPORTS = {
    "dsa_compress": (c_i32, [ctypes.POINTER(CompressArgs), c_vp]),
    "dsa_index_topk_workspace": (ctypes.c_size_t, [ctypes.POINTER(IndexArgs)]),
    "dsa_index_topk": (c_i32, [ctypes.POINTER(IndexArgs), c_vp, ctypes.c_size_t, c_vp]),
    "dsa_sparse_attn_workspace": (ctypes.c_size_t, [ctypes.POINTER(AttnArgs)]),
    "dsa_sparse_attn": (c_i32, [ctypes.POINTER(AttnArgs), c_vp, ctypes.c_size_t, c_vp]),
    "dsa_layer_workspace": (ctypes.c_size_t, [ctypes.POINTER(LayerArgs)]),
    "dsa_layer_decode": (c_i32, [ctypes.POINTER(LayerArgs), c_vp, ctypes.c_size_t, c_vp]),
    "dsa_layer_prefill": (c_i32, [ctypes.POINTER(LayerArgs), c_vp, ctypes.c_size_t, c_vp]),
    "dsa_layer_decode_noalloc": (c_i32, [ctypes.POINTER(LayerArgs), c_vp]),
    "dsa_layer_decode_noalloc_capacity": (ctypes.c_size_t, []),
    "dsa_set_timing_events": (None, [ctypes.POINTER(TimingEvents)]),
    "dsa_device_supported": (ctypes.c_int, [ctypes.c_int]),
    "dsa_version": (ctypes.c_char_p, []),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_n_complete": (c_i64, [c_i64, c_i32, c_i32]),
    "dsa_abi_sizeof": (ctypes.c_size_t, [ctypes.c_char_p]),
}
for _name, (_res, _args) in EXPORTS.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args

STRUCTS = {"dsa_timing_events": TimingEvents, "dsa_geom": Geom, "dsa_paging": Paging, "dsa_compress_args": CompressArgs, "dsa_index_args": IndexArgs,
           "dsa_attn_args": AttnArgs, "dsa_layer_args": LayerArgs}
for _n, _s in STRUCTS.items():
    if _lib.dsa_abi_sizeof(_n.encode()) != ctypes.sizeof(_s):
        raise ImportError(f"ABI mismatch for {_n}: C {_lib.dsa_abi_sizeof(_n.encode())} "
                          f"bytes, binding {ctypes.sizeof(_s)}")


class DsaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def _check(rc):
    if rc != 0:
        raise DsaError(rc, _lib.dsa_last_error().decode())


def set_timing_events(index=(None, None), attn=(None, None)):
    """dsa_set_timing_events: HipEvent pairs (or None) for the next call made
    on this thread."""
    h = [None if e is None else e.handle for e in (*index, *attn)]
    _lib.dsa_set_timing_events(ctypes.byref(TimingEvents(*h)))


def version():
    return _lib.dsa_version().decode()


def last_error():
    return _lib.dsa_last_error().decode()


def n_complete(L, s, S):
    return int(_lib.dsa_n_complete(L, s, S))


def device_supported(device=0):
    return bool(_lib.dsa_device_supported(device))


def ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    return t.data_ptr()


def dtype_code(t):
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return DSA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ws(nbytes, device):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def geom(stride, span, dim, rope_dim=0, rope_base=10000.0, rope_pos_offset=0):
    return Geom(stride, span, dim, rope_dim, rope_base, rope_pos_offset)


# ------------------------------------------------------------------ calls
def compress(args: CompressArgs, stream=None):
    """dsa_compress (S1)."""
    _check(_lib.dsa_compress(ctypes.byref(args), _stream(stream)))


def index_topk_workspace(args: IndexArgs):
    return int(_lib.dsa_index_topk_workspace(ctypes.byref(args)))


def index_topk(args: IndexArgs, ws=None, stream=None, device="cuda"):
    """dsa_index_topk (S3 + S4); allocates the workspace if none is given."""
    if ws is None:
        ws, _ = _ws(index_topk_workspace(args), device)
    _check(_lib.dsa_index_topk(ctypes.byref(args), ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(stream)))
    return ws


def sparse_attn_workspace(args: AttnArgs):
    return int(_lib.dsa_sparse_attn_workspace(ctypes.byref(args)))


def sparse_attn(args: AttnArgs, ws=None, stream=None, device="cuda"):
    """dsa_sparse_attn (S5)."""
    if ws is None:
        ws, _ = _ws(sparse_attn_workspace(args), device)
    _check(_lib.dsa_sparse_attn(ctypes.byref(args), ptr(ws), 0 if ws is None else ws.numel(),
                                _stream(stream)))
    return ws


def layer_workspace(args: LayerArgs):
    return int(_lib.dsa_layer_workspace(ctypes.byref(args)))


def layer_decode(args: LayerArgs, ws=None, stream=None, device="cuda"):
    """dsa_layer_decode (one token per sequence)."""
    if ws is None:
        ws, _ = _ws(layer_workspace(args), device)
    _check(_lib.dsa_layer_decode(ctypes.byref(args), ptr(ws), 0 if ws is None else ws.numel(),
                                 _stream(stream)))
    return ws


def layer_decode_noalloc(args: LayerArgs, stream=None):
    """dsa_layer_decode_noalloc: the decode step on the library's static
    scratch (no workspace, nothing allocated)."""
    _check(_lib.dsa_layer_decode_noalloc(ctypes.byref(args), _stream(stream)))


def layer_decode_noalloc_capacity():
    return int(_lib.dsa_layer_decode_noalloc_capacity())


def layer_prefill(args: LayerArgs, ws=None, stream=None, device="cuda"):
    """dsa_layer_prefill (a chunk of tokens per sequence)."""
    if ws is None:
        ws, _ = _ws(layer_workspace(args), device)
    _check(_lib.dsa_layer_prefill(ctypes.byref(args), ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream)))
    return ws


# ------------------------------------------------------------- HIP events
# Timing events that the library attaches to its kernels (dsa_set_timing_events)
# are plain hipEvent_t handles from the HIP runtime.
_hip = None


def _hip_rt():
    global _hip
    if _hip is None:
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise ImportError("libamdhip64.so not found")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(c_vp)]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(c_f32), c_vp, c_vp]
        _hip.hipEventDestroy.argtypes = [c_vp]
        _hip.hipEventSynchronize.argtypes = [c_vp]
    return _hip


class HipEvent:
    """A hipEvent_t owned from Python (created with timing enabled)."""

    def __init__(self):
        self.handle = c_vp()
        if _hip_rt().hipEventCreate(ctypes.byref(self.handle)) != 0:
            raise RuntimeError("hipEventCreate failed")

    def elapsed_ms(self, end):
        ms = c_f32()
        rc = _hip_rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if _hip is not None and self.handle:
            _hip.hipEventDestroy(self.handle)
