"""The speed-of-light arithmetic the pages print, reproduced by the closed
form in persistent_megakernel_03_amd.sol (CPU only)."""

import json
import os

from persistent_megakernel_03_amd import configs, sol

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_sol.json")


def test_pages_speed_of_light_numbers():
    g = json.load(open(GOLDEN))
    per_step = g["weight_bytes_per_step"] + g["kv_bytes_per_step_8k"]
    ceiling = sol.sol_tokens_per_s(per_step, 1, g["hbm_bytes_per_s"])
    p = g["printed"]
    assert abs(ceiling - 471.83) < 0.01                      # "around 470"
    assert abs(ceiling - p["ceiling_tok_s_approx"]) / p["ceiling_tok_s_approx"] < 0.01
    assert round(100 * p["megakernel_tok_s"] / ceiling) == p["megakernel_frac_pct"]
    assert round(100 * p["vllm_tok_s"] / ceiling) == p["vllm_frac_pct"]
    assert round(p["megakernel_tok_s"] / p["vllm_tok_s"], 2) == p["speedup"]


def test_closed_form_for_the_30b_shape():
    d = configs.A3B
    b = sol.step_bytes(d, [8192], [8] * 48)
    # dense attention/router/norm weights, 8 routed experts per layer, LM head,
    # final norm, one embedding row, 8193 KV positions read, one written, logits
    dense = 48 * 2 * (2048 * 5120 + 4096 * 2048 + 128 * 2048 + 2 * 2048)
    experts = 48 * 8 * 3 * 768 * 2048 * 2
    head = 151936 * 2048 * 2 + 2048 * 2 + 2048 * 2
    kv = 8193 * 48 * 2 * 4 * 128 * 2 + 48 * 2 * 4 * 128 * 2
    assert b == dense + experts + head + kv + 151936 * 4 == 6889825792
    assert abs(sol.sol_tokens_per_s(b, 1) - 1161.13) < 0.01
