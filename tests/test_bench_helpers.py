"""Host-side logic of bench.py: which kernel is dominant, and when a stored
counter summary may be used (only for the kernel sources it was taken on)."""
import json
import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_dominant_kernel_threshold_matches_the_library_dispatch():
    hdr = open(os.path.join(ROOT, "include", "moe_w4a16.h")).read()
    m = re.search(r"#define MOE_TILED_MIN_TOKENS (\d+)", hdr)
    from w4a16_routed_expert_moe_amd import _lib
    assert m and int(m.group(1)) == bench.TILED_MIN_TOKENS == _lib.MOE_TILED_MIN_TOKENS
    src = open(os.path.join(ROOT, "w4a16_routed_expert_moe_amd", "csrc", "moe_gemm_tiled.hip")).read()
    assert "return T >= MOE_TILED_MIN_TOKENS && N % kTN == 0 && K <= 4096;" in src
    assert bench.dominant_kernel(1)[0] == "k_decode_token"   # the whole layer in one launch
    assert bench.dominant_kernel(2)[0] == "k_w4a16_stream"
    assert bench.dominant_kernel(383)[0] == "k_w4a16_stream"
    assert bench.dominant_kernel(384)[0] == "k_w4a16_tiled"
    assert bench.dominant_kernel(1, "fp4")[0] == "k_mxfp4_decode_token"
    assert bench.dominant_kernel(64, "fp4")[0] == "k_mxfp4_stream"
    # FP4 at 384 tokens and up: the 512-wide tiles whenever N and K allow, which
    # the layer's gate/up GEMM (N = 2 * 2048, K = 4096) does
    fw = open(os.path.join(ROOT, "w4a16_routed_expert_moe_amd", "csrc", "moe_gemm_fp4wide.hip")).read()
    assert "return p.fp4 && p.N % kFwTN == 0 && p.K % 256 == 0 && p.K <= 4096" in fw
    assert "constexpr int kFwTN = 512;" in fw
    import synth
    for w in ("prefill8k", "stack43"):
        assert (2 * synth.WORKLOADS[w]["I"]) % 512 == 0 and synth.WORKLOADS[w]["H"] % 256 == 0
    assert bench.dominant_kernel(384, "fp4")[0] == "k_mxfp4_wide"
    assert bench.dominant_kernel(1, "w4a8")[0] == "k_w4a8_decode_token"  # W4A8 in one launch too
    # below the tiled range the quantised activations go through the FP4 weight stream in bf16
    assert bench.dominant_kernel(64, "w4a8")[0] == "k_mxfp4_stream"
    assert bench.dominant_kernel(bench.TILED_MIN_TOKENS, "w4a8")[0] == "k_mx_gemm"
    # that kernel's counter summary for W4A8 is kept apart from the FP4 one
    assert bench.traffic_tag("decode64", "w4a8", "k_mxfp4_stream") == "decode64_w4a8"
    assert bench.traffic_tag("decode64", "fp4", "k_mxfp4_stream") == "decode64"
    assert bench.traffic_tag("prefill8k", "w4a8", "k_mx_gemm") == "prefill8k"


def test_stored_traffic_is_used_only_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    name, _, files = bench.dominant_kernel(1)
    assert bench.load_traffic(name, "decode1", files) is None          # no summary
    rec = {"source_hash": bench.kernel_source_hash(files), "traffic_bytes_per_launch": 123}
    with open(bench.traffic_file(name, "decode1"), "w") as f:
        json.dump(rec, f)
    assert bench.load_traffic(name, "decode1", files) == 123
    rec["source_hash"] = "0" * 16                                       # kernel changed since
    with open(bench.traffic_file(name, "decode1"), "w") as f:
        json.dump(rec, f)
    assert bench.load_traffic(name, "decode1", files) is None


def test_committed_summaries_are_well_formed():
    for f in os.listdir(os.path.join(ROOT, "profiles")):
        if f.endswith("_traffic.json"):
            rec = json.load(open(os.path.join(ROOT, "profiles", f)))
            assert rec["traffic_bytes_per_launch"] > 0
            assert 1.5 < rec["fetch_scale"] < 2.5 and 0.9 < rec["write_scale"] < 1.1
