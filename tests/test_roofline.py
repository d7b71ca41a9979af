"""Pins of the speed-of-light byte accounting against the pages' own worked numbers."""
import json
import os

from decode_megakernel_wg_amd import roofline as R
from synth import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_sol.json")))


def test_pages_sol_arithmetic():
    sol = R.sol_tokens_per_s(GOLD["weights_bytes"] + GOLD["kv_bytes_8k"], bandwidth=GOLD["hbm_bytes_per_s"])
    assert abs(sol - GOLD["sol_tok_s_about"]) / GOLD["sol_tok_s_about"] < 0.01          # 471.8 ~ "about 470"
    assert round(100 * GOLD["megakernel_tok_s"] / sol) == GOLD["megakernel_pct_of_sol"]
    assert round(100 * GOLD["vllm_tok_s"] / sol) == GOLD["vllm_pct_of_sol"]
    assert round(GOLD["megakernel_tok_s"] / GOLD["vllm_tok_s"], 2) == GOLD["megakernel_over_vllm"]


def test_full_shape_bytes_at_8k():
    s = W.FULL
    b = R.step_bytes(s, [8192], [s.top_k] * s.n_layers, 1)
    assert b == 7_340_335_104
    assert R.weight_bytes(s, [s.top_k] * s.n_layers, 1) == 6_534_930_432
    assert abs(R.sol_tokens_per_s(b) - 1089.9) < 0.1
    # the active parameter count of the synthetic shape is about 3.3B (the pages' model: 3.3B active)
    assert 3.2e9 < R.weight_bytes(s, [s.top_k] * s.n_layers, 1) / 2 < 3.4e9


def test_tiny_shape_bytes():
    s = W.TINY
    assert R.step_bytes(s, [128], [s.top_k] * s.n_layers, 1) == 6_171_648
