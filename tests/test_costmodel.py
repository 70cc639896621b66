"""The FLOP / byte counters reproduce the worked cost model printed on the
Ling-2.6-1T page (section 1) and the Ironwood peak arithmetic (golden fixture)."""
import json
import os

import pytest

from sparse_mixture_experts_moe_amd import costmodel as cm

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ling_cost_model.json")))


def test_routed_rows_per_device():
    s = G["setting"]
    assert s["tokens"] * s["top_k"] // s["devices"] == G["routed_rows_per_device"]
    assert s["local_experts"] * s["rows_per_expert"] == G["routed_rows_per_device"]


def test_ffn_flops_match_the_printed_cost_model():
    s = G["setting"]
    rows, D, I = G["routed_rows_per_device"], s["hidden"], s["intermediate"]
    assert round(cm.ffn1_flops(rows, D, I) / 1e9, 1) == G["ffn1_gflop"]
    assert round(cm.ffn2_flops(rows, D, I) / 1e9, 1) == G["ffn2_gflop"]
    assert round(cm.ffn_flops(rows, D, I) / 1e9, 1) == G["routed_gflop"]
    # the page runs the shared expert on the 4096 local rows
    assert round(cm.ffn_flops(4096, D, I) / 1e9, 1) == G["shared_gflop"]
    total = cm.ffn_flops(rows, D, I) + cm.ffn_flops(4096, D, I)
    assert round(total / 1e9, 1) == G["total_gflop"]
    comp_ms, _ = cm.bound_ms(total, 0, G["fp8_peak_tflops_per_device"])
    assert round(comp_ms, 2) == G["compute_bound_ms"]


def test_weight_bytes_and_hbm_bounds():
    s = G["setting"]
    per = cm.expert_weight_bytes(s["hidden"], s["intermediate"], "fp8")
    assert round(per / 1e6, 1) == G["fp8_expert_mb"]
    total = s["local_experts"] * per
    # 8 x 50.3 MB: the page prints the product truncated to whole MB
    assert int(total / 1e6) == G["fp8_local_experts_mb"]
    _, ms = cm.bound_ms(0, total, 1, peak_gbs=G["hbm_tbs_per_device"] * 1000)
    assert round(ms, 2) == G["hbm_bound_ms"]
    tiles = -(-s["rows_per_expert"] // s["token_tile_bts"])
    assert tiles == 4
    assert round(tiles * ms, 2) == G["hbm_bound_ms_token_tiles"]


def test_scatter_payload():
    s = G["setting"]
    n = G["routed_rows_per_device"] * s["hidden"]
    assert n == G["scatter_elements"]
    assert round(n * 2 / 1e6, 1) == G["scatter_mb_bf16"]
    # 33.55 MB, printed truncated to one decimal
    assert int(n / 1e5) / 10 == G["scatter_mb_fp8"]


def test_peak_arithmetic():
    tf = G["mxu_flop_per_cycle"] * G["tc_ghz"] * 1e9 * G["mxu_per_chip"] / 1e12
    assert round(tf) == G["bf16_tflops_per_chip"]


def test_layer_flops_per_token():
    from workloads import CONFIGS
    per_tok = {n: cm.layer_flops(c) / c.T for n, c in CONFIGS.items()}
    assert round(per_tok["qwen_decode"] / 1e6, 1) == 281.0
    assert round(per_tok["qwen_prefill"] / 1e6, 1) == 281.0
    assert round(per_tok["gemma"] / 1e6, 1) == 131.6
    assert round(per_tok["ling_prefill"] / 1e6, 1) == 910.2
