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


def test_projection_bytes_by_hand():
    from decode_attention_absorbed_amd import accounting as acc

    # dsv3 step: 32 query rows, 128 heads
    w = 128 * 128 * 512 * 2  # one of W_UK / W_UV: 16.8 MB
    assert acc.up_project_bytes(32, 128) == w + 32 * 128 * (512 * 4 + 128 * 2)
    per_head = 32 * 128 * (128 * 2 + 512 * 2 + 2 * 64 * 2)  # q_nope in, q_abs out, q_pe in + out
    per_token = 32 * ((512 + 64) * 2 + 1152 + 64 * 4 + 4 + 4)  # c_kv + k_pe in, row out, table row, len, page id
    assert acc.prolog_bytes(32, 128) == w + per_head + per_token + 512 * 2
    assert acc.prolog_bytes(32, 128, "fp8") == acc.prolog_bytes(32, 128) - 32 * (1152 - 577)
    assert acc.o_project_bytes(32, 128) == 7168 * 16384 * 2 + 32 * (16384 + 7168) * 2  # 236.4 MB
    assert round(acc.o_project_bytes(32, 128) / 1e6, 1) == 236.4
