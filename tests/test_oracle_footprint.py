"""Pins for the oracle's footprint arithmetic against numbers the pages print (no GPU)."""
import json
import os

import pytest

from oracle import kvq_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "footprint.json")))


def test_int4_codes_are_a_quarter_of_fp16():
    fp16 = O.fp16_kv_bytes(26, 1, 256, 4096)
    q = O.quantized_kv_bytes(26, 1, 256, 4096, 4, 4, with_scales=False)
    assert q / fp16 == GOLD["int4_codes_fraction_of_fp16"]["value"]


def test_k8v4_is_one_and_a_half_bytes_per_element():
    L, H, d, S = 26, 1, 256, 4096
    q = O.quantized_kv_bytes(L, H, d, S, 8, 4, with_scales=False)
    assert q == L * H * d * S * GOLD["k8v4_bytes_per_kv_element"]["value"]


def test_48_layer_fp16_footprint():
    g = GOLD["fp16_kv_48L_16H_d128"]
    b16 = O.fp16_kv_bytes(g["layers"], g["kv_heads"], g["head_dim"], 16384)
    b32 = O.fp16_kv_bytes(g["layers"], g["kv_heads"], g["head_dim"], 32768)
    assert b16 == 6_442_450_944
    assert round(b16 / 2**30) == g["ctx_16k_gb_approx"]
    assert round(b32 / 2**30) == g["ctx_32k_gb_approx"]


@pytest.mark.parametrize("kb,vb,key", [(8, 8, "k8v8_mb"), (8, 4, "k8v4_mb"), (4, 4, "k4v4_mb")])
def test_kvsplit_table_under_32_group_accounting(kb, vb, key):
    t = GOLD["kvsplit_memory_table_8k"]
    ratio = O.quantized_kv_bytes(1, 1, 128, 8192, kb, vb, group=32) / O.fp16_kv_bytes(1, 1, 128, 8192)
    assert abs(t["fp16_mb"] * ratio - t[key]) < 1e-9


def test_our_int4_format_sits_inside_the_reported_compression_range():
    c = GOLD["compression_range"]
    ours = O.fp16_kv_bytes(1, 1, 128, 1) / O.quantized_kv_bytes(1, 1, 128, 1, 4, 4)
    assert ours == 3.2
    assert c["low"] <= ours <= c["high"]
    top = O.fp16_kv_bytes(1, 1, 128, 1) / O.quantized_kv_bytes(1, 1, 128, 1, 4, 4, group=32)
    assert abs(top - c["high"]) < 0.01
