"""The hardware fact behind the prefill indexer's exact Top-k.

The prefill path scores candidates approximately on the gfx950 scaled fp8
matrix cores and rescores only the entries an error bound cannot exclude;
the bound needs the fp8 product of a 128-term dot product to err by at most
2^-10 ||a|| ||b|| (in the operands' own units).  The pages give the indexer
in FP8 ("DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" 4.1) but no
error figure for any hardware, so this is checked here on the instruction
itself (tests/hw/fp8_mfma_probe.hip, the same builtin, operand layout and
per-row E8M0 scale form as the prefill kernel), against exact fp64 sums,
on code patterns chosen to stress its alignment:

* one maximal product plus 127 same-sign products swept in fine steps from
  equal magnitude down to 2^-26 of it (the alignment cut);
* the same with the small products of the other sign;
* cancelling sums (alternating signs);
* heavy-tailed codes, all-subnormal mixes with a few large codes, all
  +-448, and uniformly random finite codes.

It also checks that the E8M0 scale is exact: a result with scale 2^-c is
bit for bit the unscaled result times 2^-c.  The largest error ratio seen
is printed and recorded with the session's parity errors.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import codecs

from gpu_helpers import note_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
PROBE = os.path.join(os.path.dirname(__file__), "hw", "libfp8_mfma_probe.so")
BOUND = 2.0 ** -10


def _probe():
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is missing: build with python -m sparse_long_context_c4a_amd.build")
    lib = ctypes.CDLL(PROBE)
    lib.fp8_mfma_probe.restype = ctypes.c_int
    lib.fp8_mfma_probe.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    return lib


def _codes(v):
    return codecs.fp8_encode(np.asarray(v, np.float64))


def _tiles():
    """Pattern tiles: a [P, 16, 128] and b [P, 16, 128] e4m3fn codes."""
    rng = np.random.default_rng(2026)
    A, B = [], []
    # 1, 2: one product of 448^2 and 127 small ones at 2^-(x_h + y_e) of it
    for sign in (1.0, -1.0):
        for u in range(14):
            a = np.zeros((16, 128))
            b = np.zeros((16, 128))
            for i in range(16):
                xa = u + i / 16.0        # octaves below 448, rows
                xb = (i / 16.0) + 0.03   # columns add a finer offset
                a[i, 0] = 448.0
                a[i, 1:] = sign * 448.0 * 2.0 ** -xa
                b[i, 0] = 448.0
                b[i, 1:] = 448.0 * 2.0 ** -xb
            A.append(_codes(a))
            B.append(_codes(b))
    # 3: cancelling sums
    for _ in range(8):
        a = rng.standard_normal((16, 128)) * 64
        b = np.abs(rng.standard_normal((16, 128))) * 64
        b[:, 1::2] *= -1
        A.append(_codes(a))
        B.append(_codes(b))
    # 4: heavy-tailed
    for _ in range(16):
        A.append(_codes(rng.standard_normal((16, 128)) * np.exp(1.5 * rng.standard_normal((16, 128)))))
        B.append(_codes(rng.standard_normal((16, 128)) * np.exp(1.5 * rng.standard_normal((16, 128)))))
    # 5: subnormal codes with a few large ones
    for _ in range(8):
        ca = rng.integers(1, 8, (16, 128)) | (rng.integers(0, 2, (16, 128)) << 7)
        cb = rng.integers(1, 8, (16, 128)) | (rng.integers(0, 2, (16, 128)) << 7)
        big = rng.random((16, 128)) < 0.02
        ca = np.where(big, 0x70 | rng.integers(0, 7, (16, 128)), ca)
        A.append(ca.astype(np.uint8))
        B.append(cb.astype(np.uint8))
    # 6: all +-448
    for _ in range(4):
        A.append(np.where(rng.random((16, 128)) < 0.5, 0x7E, 0xFE).astype(np.uint8))
        B.append(np.where(rng.random((16, 128)) < 0.5, 0x7E, 0xFE).astype(np.uint8))
    # 7: uniform over the finite codes
    for _ in range(16):
        ca = rng.integers(0, 256, (16, 128))
        cb = rng.integers(0, 256, (16, 128))
        ca = np.where((ca & 0x7F) == 0x7F, 0x7E, ca)
        cb = np.where((cb & 0x7F) == 0x7F, 0x7E, cb)
        A.append(ca.astype(np.uint8))
        B.append(cb.astype(np.uint8))
    return np.stack(A), np.stack(B)


def _scale_codes(av, bv):
    """The prefill kernel's rule: 2^c >= 2 ||a_h|| kappa, kappa = max_e ||b_e||,
    as the E8M0 code 127 - c of 2^-c (code 127 = 1 for a zero row)."""
    na = np.sqrt((av * av).sum(axis=2))                       # [P, 16]
    kap = np.sqrt((bv * bv).sum(axis=2)).max(axis=1)          # [P]
    x = 2.0 * na * kap[:, None] * (1.0 + 2.0 ** -20)
    c = np.where(x > 0, np.frexp(np.where(x > 0, x, 1.0))[1], 0)
    return (127 - c).astype(np.int32)


def _run(lib, a, b, code):
    P = a.shape[0]
    assert a.shape == b.shape == (P, 16, 128) and code.shape == (P, 16)
    ta = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    tb = torch.from_numpy(np.ascontiguousarray(b)).to(DEV)
    tc = torch.from_numpy(np.ascontiguousarray(code)).to(DEV)
    out = torch.zeros((P, 16, 16), dtype=torch.float32, device=DEV)
    rc = lib.fp8_mfma_probe(ta.data_ptr(), tb.data_ptr(), tc.data_ptr(), out.data_ptr(), P,
                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def test_fp8_mfma_error_within_the_prefill_bound():
    lib = _probe()
    a, b = _tiles()
    print(f"[fp8 mfma probe] {a.shape[0]} tiles of 16 x 16 dot products", flush=True)
    av, bv = codecs.fp8_decode(a), codecs.fp8_decode(b)
    assert np.all(np.isfinite(av)) and np.all(np.isfinite(bv))
    code = _scale_codes(av, bv)
    got = _run(lib, a, b, code)
    # exact: every product is a multiple of 2^-18 below 2^18, a 128-term sum
    # is a multiple of 2^-18 below 2^25 (43 bits), exact in fp64
    exact = np.einsum("pik,pjk->pij", av, bv)
    sc = np.ldexp(1.0, code - 127)[:, :, None]                 # 2^-c per row
    norm = np.sqrt((av * av).sum(axis=2))[:, :, None] * np.sqrt((bv * bv).sum(axis=2))[:, None, :]
    err = np.abs(got - exact * sc)
    ratio = np.where(norm > 0, err / np.maximum(norm * sc, 1e-300), 0.0)
    worst = float(ratio.max())
    p, i, j = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    print(f"[fp8 mfma probe] worst |err| / (2^-c |a| |b|) = {worst:.3e} = 2^{np.log2(max(worst, 1e-300)):.2f}"
          f" at tile {p} ({i}, {j})", flush=True)
    note_err("fp8 mfma |err|/(|a||b|)", worst, BOUND, f"tile {p} ({i}, {j})")
    assert np.all(err[norm == 0] == 0)
    assert worst <= BOUND, f"fp8 MFMA error {worst:.3e} exceeds 2^-10 of |a||b|"


def test_fp8_mfma_e8m0_scale_is_exact():
    lib = _probe()
    a, b = _tiles()
    av, bv = codecs.fp8_decode(a), codecs.fp8_decode(b)
    code = _scale_codes(av, bv)
    one = np.full_like(code, 127)
    got_c = _run(lib, a, b, code)
    got_1 = _run(lib, a, b, one)
    sc = np.ldexp(1.0, code - 127)[:, :, None]
    want = got_1 * sc
    # where the scaled value stays a normal f32 the scale is a pure exponent shift
    normal = np.abs(want) >= 2.0 ** -126
    assert np.array_equal(got_c[normal], want[normal])
