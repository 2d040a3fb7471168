"""Host-side accounting (FLOPs and bytes the benchmark divides by), pinned to
the tables the pages print and to the oracle's own mask counts."""
import json
import os

import numpy as np
import pytest

import oracle
from global_muse_rope_amd import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def test_flop_and_byte_units():
    f = GOLD["decode_attention_gflop"]["flop_per_key_layer"]
    assert acc.flops_per_pair(128, 64) == f["spark"]
    assert acc.flops_per_pair(32, 128) == f["glimmer"]
    b = GOLD["kv_bytes_per_token_layer"]
    assert acc.kv_bytes_per_token(16, 64) == b["spark"]
    assert acc.kv_bytes_per_token(2, 128) == b["glimmer"]


@pytest.mark.parametrize("model,hq,hkv,d,ng,nl", [("spark", 128, 16, 64, 16, 46), ("glimmer", 32, 2, 128, 13, 39)])
def test_decode_attention_flops_table(model, hq, hkv, d, ng, nl):
    for c, gflop in GOLD["decode_attention_gflop"][model].items():
        got = acc.decode_attention_flops_per_token(hq, d, ng, nl, int(c)) / 1e9
        assert round(got, 1) == gflop


@pytest.mark.parametrize("model,hkv,d,ng,nl", [("spark", 16, 64, 16, 46), ("glimmer", 2, 128, 13, 39)])
def test_kv_cache_table(model, hkv, d, ng, nl):
    for c, gib in GOLD["kv_cache_gib"][model].items():
        got = acc.kv_cache_bytes(hkv, d, ng, nl, int(c)) / 2 ** 30
        assert round(got, 3) == gib


def test_pairs_match_oracle_mask():
    for n, w in [(1, 0), (2, 1), (50, 7), (129, 64), (256, 300)]:
        assert acc.visible_pairs(n, w) == int(oracle.visible_mask(n, w).sum())


def test_decode_history():
    # global: every earlier token; local: the last W - 1 earlier tokens
    assert acc.decode_visible_history(1, 0) == 0
    assert acc.decode_visible_history(100, 0) == 99
    assert acc.decode_visible_history(100, 2048) == 99
    assert acc.decode_visible_history(5000, 2048) == 2047
    for L in [1, 2, 7, 8, 9, 40]:
        lo, hi = oracle.visible_range(L - 1, 8)
        assert acc.decode_visible_history(L, 8) == hi - lo
