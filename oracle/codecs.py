"""Storage-format codecs for the oracle (bf16 and OCP fp8 e4m3fn), in fp64.

Test infrastructure only (see the package docstring).

The pages fix the *kind* of storage: bf16 for prefill KV and token-wise fp8
for the indexer ("DeepSeek V4 稀疏注意力完全解剖", 第三层 "多种量化";
"DeepSeek DSA ...详解", 4.1 Lightning Indexer: the indexer can run in FP8).
They do not spell out the bit formats, so these follow the published format
definitions:

* bf16: IEEE-754 binary32 with the low 16 fraction bits dropped (1 sign,
  8 exponent bits with bias 127, 7 fraction bits).  Encoding rounds to
  nearest, ties to even, from the exact fp64 value.
* fp8 e4m3fn (OCP 8-bit floating point specification): 1 sign, 4 exponent
  bits with bias 7, 3 fraction bits, no infinities, the single NaN pattern
  S.1111.111 per sign, largest finite magnitude 448, smallest subnormal 2^-9.
  Encoding rounds to nearest, ties to even, and saturates to +-448.
* fp4 e2m1 (OCP Microscaling Formats (MX) specification, FP4 element type):
  1 sign, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1,
  1.5, 2, 3, 4, 6; no infinities or NaN.  Encoding rounds to nearest, ties to
  the even code, and saturates to +-6; a negative value that rounds to zero
  keeps its sign (code 8).  The MX block scale (E8M0, 2^(e-127)) is in
  ``oracle.dsa.quantize_mxfp4``.

Pins (tests/test_oracle_codecs.py): every one of the 256 fp8 codes against
torch's float8_e4m3fn decode, the format's landmark values (448, 2^-6, 2^-9,
1.0), exhaustive round-trip of all finite codes, midpoint ties, and bf16
against torch's bfloat16 conversion on random and edge values; the 16 fp4
codes against the E2M1 magnitudes written out, every midpoint tie and the
saturation by hand, fp4 encoding against brute-force nearest search, and the
MX block-scale rule on hand-computed blocks.
"""

import numpy as np

FP8_MAX = 448.0
FP4_MAX = 6.0
# E2M1 magnitudes of codes 0..7 (OCP MX FP4: 1 sign, 2 exponent bits with
# bias 1, 1 mantissa bit; no infinities or NaN)
FP4_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def bf16_decode(bits):
    """uint16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _round_half_even(x):
    # numpy's rint rounds half to even
    return np.rint(x)


def bf16_encode(x):
    """float64 values -> uint16 bf16 bit patterns, round-to-nearest-even.

    Done in exact arithmetic: find the binade of |x|, scale so that one bf16
    unit in the last place is 1, round half to even, then rebuild the value
    and take its binary32 bit pattern (which has zero low bits by
    construction).  Overflow goes to infinity, as IEEE rounding does.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, exp = np.frexp(a)  # a = mant * 2**exp, mant in [0.5, 1)
    e = np.maximum(exp - 1, -126)  # below the normal range the spacing stays 2**-133
    ulp = np.ldexp(1.0, e - 7)
    with np.errstate(invalid="ignore", over="ignore"):
        q = _round_half_even(a / ulp) * ulp
        q = np.where(q >= 2.0 ** 128, np.inf, q)
        q = np.where(np.isfinite(a), q, a)  # inf stays inf, NaN stays NaN
    q = np.copysign(q, x)
    f32 = q.astype(np.float32)  # exact: every q is representable in bf16
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def fp8_decode(codes):
    """uint8 e4m3fn codes -> float64 values (NaN for the NaN pattern)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = c & 0x7
    sub = f * 2.0 ** -9
    nor = (1.0 + f / 8.0) * np.exp2(e - 7.0)
    val = np.where(e == 0, sub, nor)
    val = np.where((e == 15) & (f == 7), np.nan, val)
    return sign * val


def fp8_encode(x):
    """float64 values -> uint8 e4m3fn codes, round-to-nearest-even, saturating.

    The grid of representable magnitudes is spaced 2^-9 below 2^-6
    (subnormals and the first binade share that spacing) and 2^(e-3) in the
    binade [2^e, 2^(e+1)).  Magnitudes that round above 448 saturate to 448.
    NaN maps to the positive NaN pattern.
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    xs = np.where(nan, 0.0, x)
    sign = np.where(np.signbit(xs), 0x80, 0).astype(np.int64)
    a = np.abs(xs)
    _, exp = np.frexp(a)
    e = np.maximum(exp - 1, -6)
    step = np.ldexp(1.0, e - 3)
    q = np.minimum(_round_half_even(a / step) * step, FP8_MAX)
    # rebuild the code field by field from the rounded magnitude
    _, ex2 = np.frexp(q)
    ee = ex2 - 1
    normal = q >= 2.0 ** -6
    frac_n = np.rint((q / np.ldexp(1.0, np.where(normal, ee, 0)) - 1.0) * 8).astype(np.int64)
    code_n = ((ee + 7) << 3) | frac_n
    code_s = np.rint(q / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = np.where(nan, 0x7F, sign | code)
    return code.astype(np.uint8)


def fp4_decode(codes):
    """E2M1 codes (uint8, values 0..15; bit 3 the sign) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c & 8, -1.0, 1.0) * FP4_GRID[c & 7]


def fp4_encode(x):
    """float64 values -> E2M1 codes (uint8 0..15): the nearest magnitude of
    the grid, a tie to the even code (the grid's codes alternate mantissa
    bits 0, 1), saturating at 6; the sign bit is set for negative inputs."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), FP4_MAX)
    d = np.abs(a[..., None] - FP4_GRID)          # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    tie = d == best
    # among equally near magnitudes take the even code
    even = tie & (np.arange(8) % 2 == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(tie, axis=-1))
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)
