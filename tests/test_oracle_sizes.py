"""Pins for oracle/sizes.py against numbers the pages print
(tests/golden/pages_numbers.json, each entry citing its page and section)."""
import json
import os

import pytest

from oracle import sizes

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
H, I = 2048, 768          # 3*H*I = 4,718,592 parameters per expert
L, E, K_TOP = G["model_shape"]["moe_layers"], G["model_shape"]["experts"], G["model_shape"]["top_k"]


def test_expert_bytes_match_pages():
    assert sizes.expert_bytes("int4", H, I) == 2_433_024
    assert sizes.expert_bytes("fp8", H, I) == 4_719_744
    assert sizes.expert_bytes("bf16", H, I) == 9_437_184
    assert round(sizes.expert_bytes("int4", H, I) / 1e6, 2) == G["expert_mb"]["int4"]
    assert round(sizes.expert_bytes("fp8", H, I) / 1e6, 2) == G["expert_mb"]["fp8"]


def test_int4_with_zero_points_would_not_match():
    """Adding 4-bit zero points per group changes the MB figure: the pages'
    2.43 MB pins the symmetric (no zero point) reading."""
    groups = 2 * I * (H // 128) + H * (I // 128)
    assert round((sizes.expert_bytes("int4", H, I) + groups // 2) / 1e6, 2) != G["expert_mb"]["int4"]


def test_slot_bytes_match_pages():
    assert round(sizes.slot_bytes("int4", H, I, L) / 1e6) == G["slot_mb_48_layers"]["int4"]
    assert round(sizes.slot_bytes("fp8", H, I, L) / 1e6) == G["slot_mb_48_layers"]["fp8"]


def test_all_miss_bytes_and_needed_rate():
    assert L * K_TOP == G["activations_per_token"]["value"]
    for fmt in ("int4", "fp8"):
        b = sizes.all_miss_bytes_per_token(sizes.expert_bytes(fmt, H, I), L, K_TOP)
        assert round(b / 1e9, 2) == G["all_miss_gb_per_token"][fmt]
    r = G["fp8_rate"]
    assert round(1000 / r["tok_s"], 1) == r["ms_per_token"]
    need = sizes.link_rate_needed(G["all_miss_gb_per_token"]["fp8"] * 1e9, r["tok_s"])
    assert round(need / 1e9) == r["needed_gb_s"]
    assert need > r["pcie5_x16_gb_s"] * 1e9


def test_miss_rate_bounds_match_pages():
    mb = G["miss_bounds"]
    fp8_all = G["all_miss_gb_per_token"]["fp8"] * 1e9
    int4_all = G["all_miss_gb_per_token"]["int4"] * 1e9
    c = mb["fp8_k40"]
    assert round(100 * sizes.max_miss_rate(c["tok_s"], mb["effective_link_gb_s"] * 1e9, fp8_all)) == c["max_miss_pct"]
    assert round(100 * sizes.uniform_miss_rate(c["resident"], E)) == c["uniform_miss_pct"]
    c = mb["laptop_int4_k26"]
    pcie4_x8 = 16e9 * 8 / 8 * 128 / 130          # 16 GT/s x 8 lanes, 128b/130b
    assert round(100 * sizes.max_miss_rate(c["tok_s"], pcie4_x8, int4_all)) == c["max_miss_pct"]
    assert round(100 * sizes.uniform_miss_rate(c["resident"], E)) == c["uniform_miss_pct"]
    c = mb["desktop_int4_k92"]
    assert round(100 * sizes.max_miss_rate(c["tok_s"], c["link_gb_s"] * 1e9, int4_all)) == c["max_miss_pct"]
    assert sizes.max_miss_rate(c["tok_s"], c["link_gb_s"] * 1e9, int4_all) > sizes.uniform_miss_rate(c["resident"], E)


def test_slot_bytes_vs_kv_tokens():
    kv = G["kv"]
    per = kv["bytes_per_token_bf16"]
    assert per == 96 * 1024
    int4_slot = sizes.slot_bytes("int4", H, I, L)
    fp8_slot = sizes.slot_bytes("fp8", H, I, L)
    assert round(int4_slot / per, -1) == kv["int4_slot_tokens"]
    assert round(fp8_slot / per, -2) == kv["fp8_slot_tokens"]
    assert round(10 * int4_slot / per, -2) == kv["k_minus_10_tokens"]
    assert round(kv["cache_tokens"] * per / 1e9, 1) == kv["cache_gb"]


def test_choosing_k_example_fits():
    ex = G["choosing_k_example"]
    slot = sizes.slot_bytes("int4", H, I, L)
    budget = ex["gpu_gb"] * 1e9 * ex["mem_fraction_static"]
    assert ex["resident"] * slot < budget
    assert sizes.suggest_k(ex["resident"] * slot, slot, E) == ex["resident"]
    assert sizes.suggest_k(1e15, slot, E) == E


def test_int8_expert_bytes_equal_the_canonical_tensors():
    """No page value for int8: the closed form against the bytes of the synthetic
    canonical tensors (codes one byte per weight, fp16 per 128 inputs per row)."""
    import synth
    for H, I in ((2048, 768), (256, 128)):
        wl = synth.workload("decode_int8_k40_b4", hidden=H, inter=I)
        total = sum(t.nbytes for t in synth.expert_tensors(wl, 0, 3))
        assert sizes.expert_bytes("int8", H, I) == total
    assert sizes.expert_bytes("int8", 2048, 768) == 4_792_320


def test_mxfp4_expert_bytes_equal_the_canonical_tensors():
    """MXFP4 (OCP): 4-bit codes plus one E8M0 byte per 32 inputs per row.  At
    the gpt-oss-20b expert shape (hidden = inter = 2880) that is 3 x 2880 x 2880
    / 2 code bytes and 3 x 2880 x 90 scale bytes, with no padding: the slot
    holds exactly the host layout."""
    import synth
    for H, I in ((2880, 2880), (256, 128)):
        wl = synth.workload("decode_mxfp4_k16_b1", hidden=H, inter=I)
        total = sum(t.nbytes for t in synth.expert_tensors(wl, 0, 3))
        assert sizes.expert_bytes("mxfp4", H, I) == total
    assert sizes.expert_bytes("mxfp4", 2880, 2880) == 12_441_600 + 777_600
