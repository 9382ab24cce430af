"""Pins of entry counts, visibility and the window against the pages' figures
(tests/golden/page_figures.json) and brute-force enumeration."""

import json
import os

import numpy as np
import pytest

from oracle import dsa

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _tokens_of_entry(j, s, S, L):
    """Which raw tokens entry j mixes, found by probing the oracle compressor
    with one-hot token vectors (token p is e_p) and uniform logits."""
    eye = np.eye(L)
    c = dsa.compress_range(lambda p: eye[p], np.zeros((1, S)), j, 1, s, S, r=0, base=1.0)[0]
    return sorted(np.nonzero(c > 0)[0].tolist())


def test_c4a_group_diagram():
    g = GOLD["c4a_group_diagram"]
    for j, toks in g["entries"].items():
        assert _tokens_of_entry(int(j), g["stride"], g["span"], 64) == toks


def test_c128a_group():
    g = GOLD["c128a_group"]
    for j, (lo, hi) in g["entries"].items():
        assert _tokens_of_entry(int(j), g["stride"], g["span"], 512) == list(range(lo, hi + 1))


def test_entries_at_1m():
    g = GOLD["entries_at_1M"]
    L = g["context"]
    assert dsa.n_slots(L, 4) == g["c4a_slots"]
    assert dsa.n_slots(L, 128) == g["c128a_slots"]
    # complete c4a entries: the last slot (tokens L-4 .. L+3) is not complete
    assert dsa.n_complete(L, 4, 8) == g["c4a_slots"] - 1
    assert dsa.n_complete(L, 128, 128) == g["c128a_slots"]
    assert abs(dsa.n_complete(L, 4, 8) - g["c4a_about"]) / g["c4a_about"] < 0.05


def test_block_of_256():
    g = GOLD["block_of_256"]
    assert dsa.n_slots(g["raw"], 4) == g["c4a"]
    assert dsa.n_slots(g["raw"], 128) == g["c128a"]


@pytest.mark.parametrize("s,S", [(4, 8), (128, 128), (2, 2), (3, 7)])
def test_n_vis_brute_force(s, S):
    for m in range(0, 1200 if s < 100 else 4096):
        brute = sum(1 for j in range(m + 1) if s * j + S - 1 < m)
        assert dsa.n_vis(m, s, S) == brute


def test_first_c128a_entry_invisible_to_early_queries():
    # P2 机制四: the first c128a entry covers 0..127; queries up to 127 see no entry
    assert all(dsa.n_vis(m, 128, 128) == 0 for m in range(128))
    assert dsa.n_vis(128, 128, 128) == 1
    # floor division: small m must not produce a phantom entry
    assert dsa.n_vis(3, 4, 8) == 0 and dsa.n_vis(7, 4, 8) == 0 and dsa.n_vis(8, 4, 8) == 1


def test_decode_positions_of_the_workloads():
    assert dsa.n_vis(1023, 4, 8) == 254
    assert dsa.n_vis(65535, 4, 8) == 16382
    assert dsa.n_vis(1048575, 4, 8) == 262142
    assert dsa.n_vis(1048575, 128, 128) == 8191
    assert dsa.n_vis(126976, 4, 8) == 31743 and dsa.n_vis(131071, 4, 8) == 32766


def test_window_brute_force():
    W = GOLD["window"]["W"]
    for m in [0, 1, 5, 127, 128, 129, 1000]:
        mask = [n for n in range(m + 5) if m - W <= n <= m - 1]
        assert list(dsa.window_range(m, W)) == mask
    assert len(dsa.window_range(0, W)) == 0
    assert len(dsa.window_range(10_000, W)) == W


def test_kv_memory_figures_are_consistent():
    """The pages' KV-size figures agree with each other: 1M tokens x 61
    layers x 1408 B is 83.9 GiB, and the per-sequence sizes of the V4 rows
    divide to their per-token averages (about 160 and 80 B) and to the
    quoted ~8.7x reduction."""
    f = GOLD["kv_memory"]
    per_layer_tokens = f["context"] * f["layers"]
    assert round(per_layer_tokens * f["v32_bytes_per_token_layer"] / 2 ** 30, 1) == \
        f["v32_gib_per_seq"]
    b4 = f["v4_bf16_gib_per_seq"] * 2 ** 30 / per_layer_tokens
    assert abs(b4 - f["v4_bf16_bytes_per_token_layer_about"]) / 160 < 0.02   # 161.5 B
    b8 = f["v4_fp4_fp8_gib_per_seq_about"] * 2 ** 30 / per_layer_tokens
    assert abs(b8 - f["v4_fp4_fp8_bytes_per_token_layer_about"]) / 80 < 0.02  # 80.6 B
    assert round(f["v32_gib_per_seq"] / f["v4_bf16_gib_per_seq"], 1) == f["compression_factor_about"]
