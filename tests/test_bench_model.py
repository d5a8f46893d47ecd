"""CPU checks of the bench's algorithmic work model (what the roofline prices)."""
import json
import os

import numpy as np

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def test_budget_and_28x_reduction_from_the_pages():
    g = json.load(open(os.path.join(HERE, "golden", "msa_budget.json")))
    assert g["block_size"] * g["topk"] == g["tokens_per_query"]
    r = bench.attention_reduction_ratio(G=8, d=128, dI=64, N=g["context"], budget=g["tokens_per_query"])
    assert abs(r - g["attention_compute_reduction_1M"]) < 0.05


def test_prefill_model_counts_the_causal_triangle():
    # T = N = 256, B = 128, k = 16 >= nb: every causal key is attended, dense causal flops
    S, T, N, H, Hkv, d, dI, k = 1, 256, 256, 8, 2, 64, 32, 16
    m = bench.prefill_model(S, T, N, H, Hkv, d, dI, k)
    causal_pairs = T * (T + 1) // 2
    assert m["idx_scores"]["flops"] == 2 * dI * Hkv * causal_pairs
    assert m["ogq_attention"]["flops"] == 4 * d * H * causal_pairs
    # partial traffic: one (d bf16 + lse) record per (t, head, valid slot)
    slots = np.minimum(k, np.arange(T) // 128 + 1).sum()
    part = Hkv * slots * (H // Hkv) * (d * 2 + 4)
    assert m["lse_merge"]["bytes"] == part + 2 * T * H * d + 4 * Hkv * T * k


def test_c2_model_magnitudes():
    m = bench.prefill_model(1, 131072, 131072, 64, 8, 128, 64, 16)
    assert abs(m["idx_scores"]["flops"] / 1e12 - 8.80) < 0.01
    assert abs(m["ogq_attention"]["flops"] / 1e12 - 8.46) < 0.01
    rf = bench.roofline(m["ogq_attention"]["flops"], m["ogq_attention"]["bytes"], 10e-3)
    assert rf["bound"] == "hbm"


def test_decode_model_index_stream():
    m = bench.decode_model(16, 1 << 20, 64, 8, 128, 64, 16)
    assert abs(m["idx_scores"]["bytes"] / 1e9 - 17.18) < 0.01
    assert bench.roofline(m["idx_scores"]["flops"], m["idx_scores"]["bytes"], 1e-3)["bound"] == "hbm"
