"""Pins of the oracle's storage codecs (bf16, OCP fp8 e4m3fn).

The fp8 grid is fixed by the OCP 8-bit floating point format definition;
torch's float8_e4m3fn and bfloat16 casts serve as an independent library
check.  The pages name the formats (token-wise fp8 indexer keys, bf16 KV:
"DeepSeek V4 稀疏注意力完全解剖", 第三层) but not their bits.
"""

import numpy as np
import pytest
import torch

from oracle import codecs


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = codecs.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def test_fp8_landmarks():
    d = lambda c: float(codecs.fp8_decode(np.array([c], np.uint8))[0])  # noqa: E731
    assert d(0x7E) == 448.0           # largest finite
    assert d(0xFE) == -448.0
    assert d(0x38) == 1.0             # exponent field 7 = bias
    assert d(0x08) == 2.0 ** -6       # smallest normal
    assert d(0x01) == 2.0 ** -9       # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9   # largest subnormal
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    # exactly 254 finite values (126 per sign plus two zeros): no infinities
    vals = codecs.fp8_decode(np.arange(256, dtype=np.uint8))
    assert np.isfinite(vals).sum() == 254


def test_fp8_encode_roundtrip_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = codecs.fp8_decode(codes)
    fin = np.isfinite(vals)
    back = codecs.fp8_encode(vals[fin])
    assert np.array_equal(codecs.fp8_decode(back), vals[fin])


@pytest.mark.parametrize("x,expect", [
    (1.0625, 1.0),        # midpoint 1 | 1.125 -> even mantissa (1.0)
    (1.1875, 1.25),       # midpoint 1.125 | 1.25 -> even (1.25)
    (1.0625 + 1e-12, 1.125),
    (464.0, 448.0),       # would round to 480 (not finite in e4m3fn): saturate
    (1e9, 448.0),
    (-1e9, -448.0),
    (2.0 ** -10, 0.0),    # midpoint 0 | 2^-9 -> even (0)
    (1.5 * 2.0 ** -10, 2.0 ** -9),
    (3 * 2.0 ** -10, 2 * 2.0 ** -9),  # midpoint of subnormals 1 and 2 -> 2
    (2.0 ** -6 * 1.0625, 2.0 ** -6),
])
def test_fp8_encode_rounding(x, expect):
    got = codecs.fp8_decode(codecs.fp8_encode(np.array([x])))[0]
    assert got == expect


def test_fp8_encode_matches_torch_in_range():
    x = np.random.default_rng(1).standard_normal(200_000).astype(np.float32) * 60
    x = np.clip(x, -448, 448)
    mine = codecs.fp8_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100_000) * 10.0,
                        rng.standard_normal(1000) * 1e-38,
                        [0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-45]]).astype(np.float32)
    mine = codecs.bf16_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(codecs.bf16_decode(mine),
                          torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())


def test_bf16_single_rounding_from_fp64():
    # 4.515625 is the midpoint of bf16 neighbours 4.5 and 4.53125; a value just
    # above it must round up.  (A cast through float32 would first land on the
    # midpoint and then tie to even, 4.5: the oracle rounds once.)
    v = 4.515625 + 1e-7
    assert codecs.bf16_decode(codecs.bf16_encode(np.array([v])))[0] == 4.53125
    assert codecs.bf16_decode(codecs.bf16_encode(np.array([4.515625])))[0] == 4.5
    assert np.isinf(codecs.bf16_decode(codecs.bf16_encode(np.array([3.5e38])))[0])


# ------------------------------------------------------------ fp4 / MXFP4
def test_fp4_every_code():
    """The 16 E2M1 codes (OCP MX FP4: sign, 2 exponent bits with bias 1, one
    mantissa bit), written out: 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = codecs.fp4_decode(np.arange(16, dtype=np.uint8))
    assert np.array_equal(got[:8], want)
    assert np.array_equal(got[8:], [-v for v in want])
    assert np.signbit(got[8])  # code 8 is -0
    assert np.array_equal(codecs.fp4_encode(np.array(want + [-v for v in want])),
                          np.arange(16, dtype=np.uint8))


def test_fp4_rounding_ties_and_saturation():
    x = np.array([0.25, 0.26, 0.74, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.01, 6.0, 7.0, 1e9,
                  -0.1, -0.25, -0.75, -2.5, -7.0])
    # midpoints go to the code with mantissa bit 0; beyond 6 saturates
    want = [0, 1, 1, 2, 2, 4, 4, 6, 6, 7, 7, 7, 7, 8, 8, 10, 12, 15]
    assert codecs.fp4_encode(x).tolist() == want


def test_fp4_nearest_by_brute_force():
    x = np.random.default_rng(5).uniform(-8, 8, 20000)
    c = codecs.fp4_encode(x)
    err = np.abs(codecs.fp4_decode(c) - np.clip(x, -6, 6))
    grid = np.concatenate([-codecs.FP4_GRID, codecs.FP4_GRID])
    best = np.min(np.abs(np.clip(x, -6, 6)[:, None] - grid[None, :]), axis=1)
    assert np.allclose(err, best, atol=0, rtol=0)


def test_mxfp4_block_scale_rule():
    """OCP MX conversion: e = floor(log2(max|block|)) - 2 for E2M1, elements
    v / 2^e rounded to E2M1 (saturating); an all-zero block gets e = -127."""
    from oracle import dsa
    blocks = np.zeros((6, 32))
    blocks[0, 3] = 6.0             # amax 6: e = 0, exact
    blocks[1, 0] = 7.0             # amax 7: e = 0, saturates to 6
    blocks[2, 5] = 8.0             # amax 8: e = 1, 8 = 4 * 2
    blocks[3, :] = 0.3             # amax 0.3: e = -4, 0.3 * 16 = 4.8 -> 4, value 0.25
    blocks[4, :4] = [-3.0, 1.5, 0.75, 0.0]  # amax 3: e = -1; -6, 3, 1.5, 0
    codes, sc = dsa.quantize_mxfp4(blocks.reshape(1, -1)[:, :32 * 6].reshape(6, 32))
    assert sc[:, 0].tolist() == [127, 127, 128, 123, 126, 0]
    dec = dsa.mxfp4_decode(codes, sc)
    assert dec[0, 3] == 6.0 and dec[1, 0] == 6.0 and dec[2, 5] == 8.0
    assert np.all(dec[3] == 0.25)
    assert dec[4, :4].tolist() == [-3.0, 1.5, 0.75, 0.0]
    assert np.all(dec[5] == 0.0) and np.all(codes[5] == 0)
    # a 128-dim vector holds 4 independent blocks
    v = np.random.default_rng(3).standard_normal(128) * np.repeat([1e-3, 1.0, 50.0, 3e4], 32)
    c4, s4 = dsa.quantize_mxfp4(v)
    assert s4.shape == (4,)
    d4 = dsa.mxfp4_decode(c4, s4)
    for i in range(4):
        blk = v[32 * i:32 * i + 32]
        x = np.ldexp(1.0, int(s4[i]) - 127)
        # at most half of the widest step (2 X) below 6 X, and up to 2 X where
        # the largest element (< 8 X) saturates to 6 X
        assert np.max(np.abs(d4[32 * i:32 * i + 32] - blk)) <= 2.0 * x
