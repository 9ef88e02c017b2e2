"""FLOP and byte accounting against the numbers the pages print (CPU only)."""
import json
import os

from decode_attention_absorbed_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")


def test_flop_convention_matches_time_model():
    g = json.load(open(GOLDEN))["mla_time_model"]
    # the page's convention: every query against all keys
    f = acc.flops([g["kv_len"]], g["heads"], g["q_len"], visible=False)
    t_us = f / (g["peak_flops"] * g["utilisation"] * g["overlap"]) * 1e6
    assert round(t_us, 1) == g["microseconds_per_request"]
    # visible-key count is lower by exactly one key of query 0
    fv = acc.flops([g["kv_len"]], g["heads"], g["q_len"], visible=True)
    assert f - fv == 2 * (576 + 512) * g["heads"]


def test_kv_bytes_match_memory_estimate():
    g = json.load(open(GOLDEN))["kv_cache_memory"]
    per_layer = acc.kv_bytes([g["seq_len"]] * g["concurrency"])
    total_gb = per_layer * g["layers"] / 1e9
    assert abs(total_gb - g["approx_gb"]) / g["approx_gb"] < 0.05  # 20.7 GB


def test_visible_keys_small_cases():
    assert acc.visible_key_count([5], 1) == 5
    assert acc.visible_key_count([5], 2) == 4 + 5
    assert acc.visible_key_count([7, 3], 3) == (5 + 6 + 7) + (1 + 2 + 3)


def test_roofline_binding_side():
    r2 = acc.roofline_seconds([4096] * 32, 128, 1, 64)
    assert r2["bound"] == "hbm"
    r3 = acc.roofline_seconds([4608] * 64, 128, 2, 64)
    assert r3["bound"] == "mfma"
