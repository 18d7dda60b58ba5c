"""The oracle's cache-size closed forms against the figures the pages print
(tests/golden/cache_sizes.json, each entry cited)."""

import json
import os

import pytest

from oracle import mla_oracle as orc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cache_sizes.json")))

L, H, DH, DC, DR, FP16 = 61, 128, 128, 512, 64, 2
GIB = 2.0 ** 30


def computed():
    mha = orc.mha_cache_bytes_per_token(DH, H, L, FP16)
    mla = orc.mla_cache_bytes_per_token(DC, DR, L, FP16)
    full_width = orc.mha_cache_bytes_per_token(7168, 1, L, FP16)  # 2 x 7168 per layer
    return {
        "mha_bytes_per_token": mha,
        "mha_100k_tokens_bytes": 100_000 * mha,
        "mla_bytes_per_token": mla,
        "mla_kib_per_token": mla / 1024,
        "mla_vs_mha_factor": mha / mla,
        "mqa_bytes_per_token": orc.mha_cache_bytes_per_token(DH, 1, L, FP16),
        "gqa8_bytes_per_token": orc.mha_cache_bytes_per_token(DH, H // 8, L, FP16),
        "gqa_equivalent_groups": orc.gqa_equivalent_groups(DC, DR, DH),
        "mla_32k_tokens_gib": 32768 * mla / GIB,
        "full_kv_32k_tokens_gib": 32768 * full_width / GIB,
        "full_kv_cut_fraction": 1 - mla / full_width,
    }


@pytest.mark.parametrize("key", [k for k in GOLD if not k.startswith("_")])
def test_closed_form(key):
    g = GOLD[key]
    v = computed()[key]
    if g.get("exact"):
        assert v == g["value"], (key, v)
    elif "approx_rel" in g:
        assert abs(v - g["value"]) <= g["approx_rel"] * g["value"], (key, v)
    else:
        assert abs(v - g["value"]) <= g["approx_abs"], (key, v)


def test_fp8_row_with_scale():
    # 576 one-byte codes + a 2-byte scale per layer
    assert orc.mla_cache_bytes_per_token(DC, DR, L, 1, scale_bytes=2) == 35258
    assert orc.mla_cache_bytes_per_token(DC, DR, 1, 2) == 1152
