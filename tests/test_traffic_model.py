"""Pins for the memory-traffic model against the page's worked example (CPU only)."""
import json
import math
import os

import pytest

from contextual_activation_sparsity_amd import traffic

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p1_traffic_example.json")))


def shown(value, digits, mode):
    f = 10 ** digits
    return math.floor(value * f) / f if mode == "trunc" else round(value, digits)


def computed():
    m = GOLD["model"]
    n, d, F, P = m["n_layers"], m["d_model"], m["d_ffn"], m["p_bytes"]
    bw = m["bandwidth_GBps"] * 1e9
    att = traffic.attn_weight_bytes_per_layer(d, P)
    mlp = traffic.mlp_weight_bytes_per_layer(d, F, P, m["n_mlp_mats"])
    dense = traffic.dense_weight_bytes_per_layer(d, F, P, m["n_mlp_mats"])
    sp = traffic.sparse_weight_bytes_per_layer(d, F, P, m["s_attn"], m["s_mlp"], m["n_mlp_mats"])
    t_dense = traffic.stream_time_lower_bound_s(n * dense, bw) * 1e3
    t_sp = traffic.stream_time_lower_bound_s(n * sp, bw) * 1e3
    return {
        "attention weight MB per layer": att / 1e6,
        "MLP weight MB per layer": mlp / 1e6,
        "dense MB per layer": dense / 1e6,
        "dense GB per token": n * dense / 1e9,
        "sparse attention MB per layer": m["s_attn"] * att / 1e6,
        "sparse MLP MB per layer": m["s_mlp"] * mlp / 1e6,
        "sparse MB per layer": sp / 1e6,
        "sparse GB per token": n * sp / 1e9,
        "traffic reduction ratio": dense / sp,
        "dense ms per token bound": t_dense,
        "sparse streaming ms per token bound": t_sp,
        "sparse ms per token incl. predictor": t_sp + m["t_pred_ms"],
        "140 GB streaming bound ms (A100)": traffic.stream_time_lower_bound_s(140e9, bw) * 1e3,
    }


@pytest.mark.parametrize("entry", GOLD["printed"], ids=lambda e: e["what"])
def test_worked_example(entry):
    got = computed()[entry["what"]]
    assert shown(got, entry["digits"], entry["mode"]) == pytest.approx(entry["value"], abs=1e-9)


def test_step_bytes_opt175b_shape():
    """Per-layer-token bytes of the OPT-175B-shaped step at 5 % / 20 %."""
    b = traffic.step_bytes(12288, 49152, 96, 128, 1000, 2048, 2458, 19, 2)
    assert b["predictor"] == (2 * 1000 * 12288 + 1000 * (49152 + 96)) * 2
    assert b["w1"] == 2458 * 12288 * 2 + 2458 * 4
    assert 527e6 < b["total"] < 528.5e6
    dense = traffic.dense_layer_bytes(12288, 49152, 96, 128, 2048, 2)
    assert 3.72e9 < dense < 3.73e9
