"""The layer shape used throughout matches the constants printed on the pages.

``tests/golden/deepseek_v4_flash_moe_shape.json`` holds each constant with its
citation.  The expert intermediate size (2048) is not on the pages; the
closed-form size checks below show it is consistent with what they print.
"""
import json
import os

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    with open(os.path.join(HERE, "golden", "deepseek_v4_flash_moe_shape.json")) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


def test_full_size_workloads_use_the_pages_layer_shape():
    g = _golden()
    for name in ("decode1", "decode64", "prefill8k", "stack43"):
        w = synth.WORKLOADS[name]
        assert w["H"] == g["hidden"]
        assert w["E"] == g["routed_experts"]
        assert w["k"] == g["top_k"]
        assert w["n_shared"] == g["shared_experts"]
    assert synth.WORKLOADS["stack43"]["layers"] == g["decoder_layers"]


def test_routed_expert_footprint_is_consistent_with_the_pages():
    g = _golden()
    I = synth.WORKLOADS["decode1"]["I"]
    params = g["decoder_layers"] * g["routed_experts"] * g["projections_per_expert"] * g["hidden"] * I
    assert params == 277_025_390_592
    assert params < g["total_params_billion"] * 1e9        # "most of the 284B parameters"
    nibble_bytes = params * g["weight_bits"] // 8
    scale_bytes = params // g["group_size"] * 2               # one fp16 per group of 128
    assert nibble_bytes == 138_512_695_296
    assert nibble_bytes + scale_bytes < g["quantized_size_GB"] * 1e9
