"""Pins of the speed-of-light arithmetic against the numbers the pages print."""
import json
import os

import pytest

from persistent_runtime_amd import sol
from synth.configs import LLAMA8B, MOE30B

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sol_pins.json")))


def test_mpk_bound_10ms():
    p = G["mpk_a100_bound"]
    t = sol.sol_seconds(p["weight_bytes"], p["bandwidth"])
    assert abs(t * 1e3 - p["bound_ms"]) < 1e-9
    assert p["mpk_ms"] / p["bound_ms"] == pytest.approx(1.25)


def test_cohere_sol_and_fractions():
    p = G["cohere_h100"]
    assert p["active_params"] * 2 == pytest.approx(p["weight_bytes"])
    tok = sol.sol_tokens_per_s(p["weight_bytes"] + p["kv_bytes"], 1, p["bandwidth"])
    assert abs(tok - p["sol_tok_s_approx"]) < 5        # 471.8
    assert round(100 * p["mk_tok_s"] / tok) == p["mk_pct"]
    assert round(100 * p["vllm_tok_s"] / tok) == p["vllm_pct"]
    assert round(p["mk_tok_s"] / p["vllm_tok_s"], 2) == p["speedup"]


def test_wave_quantization_example():
    p = G["wave_quantization"]
    assert sol.waves(p["tiles"], p["units"]) == (p["waves"], p["tail"], p["idle"])


def test_model_weight_bytes_match_pages():
    p = G["model_weight_bytes"]
    b8 = sol.weight_bytes_per_step(LLAMA8B, include_embed_table=True) / 1e9
    assert abs(b8 / p["dense8b_gb"] - 1) < p["dense8b_rel_tol"], b8
    bm = sol.weight_bytes_per_step(MOE30B, include_embed_table=True) / 1e9
    assert abs(bm / p["moe_active_gb"] - 1) < p["moe_rel_tol"], bm


def test_step_bytes_8b_batch1():
    # weights read by one batch-1 step of the 8B shape: 15.01 GB (+ KV)
    w = sol.weight_bytes_per_step(LLAMA8B)
    assert 15.00e9 < w < 15.02e9
    assert sol.kv_bytes_per_token(LLAMA8B) == 131072
    assert sol.step_bytes(LLAMA8B, [40]) == w + 40 * 131072
