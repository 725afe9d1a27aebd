"""GPU parity of the fp8-activation paths against the oracle: the activation
quantisation (bit-exact), the W4A8 layer (FP4 expert weights, e4m3
activations per token per 128; "Throughputmaxxing: DeepSeek-V4-Flash on
Isambard-AI", "A pass through the model") and the FP8_BLOCK GEMM (model card
"canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Component precisions").

Below MOE_TILED_MIN_TOKENS tokens the W4A8 layer multiplies the quantised
activations, written back in bf16 by moe_act_quant_fp8_dequant (exact), with
the FP4 weight-stream kernels; from there on it uses the block-scaled fp8
GEMM.  The shapes below take both paths.

Routing, the permutation, and the quantisation of x are bit-identical.  h is
produced by the GEMM and so differs from the oracle's by accumulation order;
h, y and the output are compared within 2e-2 of the largest reference value.
h's fp8 codes and scales are checked where the method decides them: they must
equal, bit for bit, the oracle's quantisation of the GPU's own h (a code may
sit one e4m3 step from the oracle's where the two h differ by a bf16 ulp, up
to 1/16 of the value; the distance to the oracle's codes is printed).  Each
test prints its errors and, for the layer, the gap to the same layer with
bf16 activations (the W4A8 accuracy contract).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_routed_expert_moe_amd as moe
from gpu_common import (TOL, Case, assert_routing_equal, bf16_to_np_bits, bits_to_f64, rel_err, say,
                        to_dev_bf16)

pytestmark = pytest.mark.gpu


def _deq(codes, scales):
    """e4m3 codes [n][K] with UE8M0 scales [n][K/128] -> fp64 (torch's float8 decoder)."""
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v * np.repeat(2.0 ** (scales.astype(np.float64) - 127), 128, axis=1)


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


@pytest.mark.parametrize("rows,K,spread", [(1, 128, 1.0), (37, 384, 1e3), (300, 4096, 1.0), (5, 2048, 1e30)])
def test_act_quant_bit_exact(rows, K, spread):
    rng = np.random.default_rng(rows + K)
    mag = np.exp(rng.uniform(-np.log(spread), np.log(spread), (rows, 1))) if spread > 1 else 1.0
    x = synth.f32_to_bf16_bits((rng.standard_normal((rows, K)) * mag).astype(np.float32))
    if rows > 1:
        x[1, :128] = 0                                    # a block of zeros
        x[0, 5] = 0x0001                                  # a bf16 subnormal
        x[rows - 1, -128:] = np.arange(128, dtype=np.uint16) | np.uint16(0x8000)  # a block of subnormals
    codes = torch.full((rows, K), 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, K // 128), 0xAA, dtype=torch.uint8, device="cuda")
    moe.moe_act_quant_fp8(rows, K, to_dev_bf16(x), codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.act_quant_fp8(x)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    say("  act quant %dx%d: codes and scales bit-exact" % (rows, K))


@pytest.mark.parametrize("rows,K,spread", [(1, 128, 1.0), (37, 384, 1e3), (300, 4096, 1.0), (5, 2048, 1e30)])
def test_act_quant_dequant_bit_exact(rows, K, spread):
    """moe_act_quant_fp8_dequant: the oracle's codes and scales, and each code
    times its scale, exactly, in bf16."""
    rng = np.random.default_rng(rows + K + 1)
    mag = np.exp(rng.uniform(-np.log(spread), np.log(spread), (rows, 1))) if spread > 1 else 1.0
    x = synth.f32_to_bf16_bits((rng.standard_normal((rows, K)) * mag).astype(np.float32))
    if rows > 1:
        x[1, :128] = 0                                    # a block of zeros
        x[0, 5] = 0x0001                                  # a bf16 subnormal
        x[rows - 1, -128:] = np.arange(128, dtype=np.uint16) | np.uint16(0x8000)  # a block of subnormals
        x[rows - 1, :128] = 0x7F00 + np.arange(128, dtype=np.uint16) % 3  # near the largest bf16
    codes = torch.full((rows, K), 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, K // 128), 0xAA, dtype=torch.uint8, device="cuda")
    deq = torch.full((rows, K), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    moe.moe_act_quant_fp8_dequant(rows, K, to_dev_bf16(x), codes, scales, deq)
    torch.cuda.synchronize()
    rc, rs = oracle.act_quant_fp8(x)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    ref64 = _deq(rc, rs)
    ref = ref64.astype(np.float32)
    # every reference value here is a bf16 value (the fp32 conversion and the
    # cut to 16 bits lose nothing)
    assert np.array_equal(ref.astype(np.float64), ref64) and not np.any(ref.view(np.uint32) & 0xFFFF)
    assert np.array_equal(bf16_to_np_bits(deq), (ref.view(np.uint32) >> 16).astype(np.uint16))
    say("  act quant + dequant %dx%d: codes, scales and bf16 values bit-exact" % (rows, K))


def _check_w4a8_layer(case: Case):
    out = bf16_to_np_bits(case.run())
    w13, s13, w2, s2 = case.stacked_weights()
    ref = oracle.layer_forward_w4a8(case.x, case.wr, case.bias, w13, s13, w2, s2, k=case.k, n_shared=case.ns)
    assert_routing_equal(case.gpu_routing(), ref)
    b = case.buf
    assert np.array_equal(b.xq.cpu().numpy(), oracle.act_quant_fp8(case.x)[0])
    h_gpu = bf16_to_np_bits(b.h)
    eh = rel_err(h_gpu, ref["h"])
    hq, hs = b.hq.cpu().numpy(), b.hqs.cpu().numpy()
    own_q, own_s = oracle.act_quant_fp8(h_gpu)
    assert np.array_equal(hs, own_s) and np.array_equal(hq, own_q)
    ehq = _rel(_deq(hq, hs), _deq(ref["hq"], ref["hs"]))
    ey = rel_err(bf16_to_np_bits(b.y), ref["y"])
    eo = rel_err(out, ref["out"])
    a16 = oracle.layer_forward(case.x, case.wr, case.bias, w13, s13, w2, s2, k=case.k, n_shared=case.ns,
                               fmt="fp4")
    gap = rel_err(out, a16["out"])
    say("  rel err h %.2e hq %.2e y %.2e out %.2e; vs the bf16-activation layer %.2e" % (eh, ehq, ey, eo, gap))
    assert eh <= TOL and ey <= TOL and eo <= TOL
    if 1 < case.T < moe.MOE_TILED_MIN_TOKENS:
        # the weight-stream path multiplies the same products as the
        # block-scaled GEMM: the two h differ only by fp32 summation order
        # (so by at most a bf16 rounding step here and there)
        ex, d = case.experts, case.desc
        h_mx = torch.empty_like(b.h)
        moe.moe_w4a8_grouped_gemm(d, case.T, b.xq, b.xqs, b.sorted_token, case.T, 2 * case.I, case.H, ex.w13,
                                  ex.s13, b.group_offsets, moe.MOE_ACT_SWIGLU, h_mx)
        torch.cuda.synchronize()
        e_mx = rel_err(h_gpu, bf16_to_np_bits(h_mx))
        say("  h against the block-scaled GEMM on the same codes: %.2e of max|h|" % e_mx)
        assert e_mx <= 8e-3


def test_w4a8_tiny_layer_every_element():
    _check_w4a8_layer(Case("tiny", fmt="fp4", w4a8=True, weights="host"))


@pytest.mark.parametrize("shape", [
    dict(T=37, H=1024, E=40, k=3, I=512, n_shared=1),   # ragged groups
    dict(T=5, H=512, E=8, k=8, I=128, n_shared=0),      # k = E, no shared expert
    dict(T=420, H=512, E=16, k=2, I=256, n_shared=1),   # groups over two 128-row tiles (block-scaled GEMM)
    dict(T=64, H=2048, E=8, k=2, I=1024, n_shared=1),   # K/128 = 16 and 8 (FP4 weight stream)
    dict(T=400, H=4096, E=8, k=2, I=2048, n_shared=1),  # 512-wide tiles at K = 4096 and 2048
    dict(T=300, H=512, E=16, k=2, I=256, n_shared=1),   # the weight stream just below the tiled range
    dict(T=3, H=1024, E=32, k=4, I=256, n_shared=1),    # a few tokens: the one-launch route + permute
])
def test_w4a8_shapes_every_element(shape):
    import os
    oracle.set_threads(max(1, min(16, len(os.sched_getaffinity(0)))))
    _check_w4a8_layer(Case("shape", seed=19, weights="host", fmt="fp4", w4a8=True, **shape))


@pytest.mark.parametrize("shape", [
    dict(H=2048, E=64, k=4, I=256, n_shared=1),
    dict(H=2048, E=16, k=8, I=1024, n_shared=0),
    dict(H=2048, E=128, k=6, I=1536, n_shared=1),
    dict(H=4096, E=32, k=2, I=512, n_shared=1),
])
def test_w4a8_decode_token_every_element(shape):
    # the one-launch W4A8 step: routing bit-exact, h and out within tolerance
    # of the oracle's W4A8 layer, deterministic over calls, and close to the
    # separate launches (quantise, two W4A8 grouped GEMMs, combine)
    case = Case("shape", T=1, seed=23, weights="host", fmt="fp4", w4a8=True, **shape)
    assert case.layer_obj.one_launch(1), "the device does not support this decode shape"
    outs = []
    for _ in range(3):
        outs.append(bf16_to_np_bits(case.run()).copy())
        assert case.buf.decode_ws[3].item() == 0, "a wait timed out"
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    w13, s13, w2, s2 = case.stacked_weights()
    ref = oracle.layer_forward_w4a8(case.x, case.wr, case.bias, w13, s13, w2, s2, k=case.k, n_shared=case.ns)
    assert_routing_equal(case.gpu_routing(), ref)
    eh, eo = rel_err(bf16_to_np_bits(case.buf.h), ref["h"]), rel_err(outs[0], ref["out"])
    case.layer_obj.fuse_token = False
    sep = bf16_to_np_bits(case.run()).copy()
    es = rel_err(outs[0], sep)
    say("  one launch: rel err h %.2e out %.2e; vs the separate launches %.2e" % (eh, eo, es))
    assert eh <= TOL and eo <= TOL and es <= TOL


def test_w4a8_decode_token_full_size():
    # decode1 (H 4096, 256 + 1 experts, top 6, I 2048) in one launch: routing
    # bit-exact, the token's out against the oracle's W4A8 MLPs of its groups
    case = Case("decode1", fmt="fp4", w4a8=True)
    assert case.layer_obj.one_launch(1)
    out = bf16_to_np_bits(case.run())
    assert case.buf.decode_ws[3].item() == 0, "a wait timed out"
    ref = case.oracle_routing()
    assert_routing_equal(case.gpu_routing(), ref)
    exp = oracle.token_outputs([0], case.x, ref["idx"], ref["w"], case.group_weights, case.E, case.ns, fmt="w4a8")
    e = rel_err(out[[0]], exp)
    say("  decode1 W4A8 one launch: out rel err %.2e" % e)
    assert e <= TOL


def _w4a8_groups(case: Case, ref, groups):
    off, st = ref["offsets"], ref["sorted_token"]
    h_all, y_all = bf16_to_np_bits(case.buf.h), bf16_to_np_bits(case.buf.y)
    worst = 0.0
    for g in groups:
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        h_ref, _, _, y_ref = oracle.expert_mlp_w4a8(case.x[st[lo:hi]], *case.group_weights(g))
        eh, ey = rel_err(h_all[lo:hi], h_ref), rel_err(y_all[lo:hi], y_ref)
        say("  group %d (%d rows): h rel err %.2e, y rel err %.2e" % (g, hi - lo, eh, ey))
        assert eh <= TOL and ey <= TOL
        worst = max(worst, eh, ey)
    return worst


@pytest.mark.parametrize("name,layer", [("prefill8k", 0), ("stack43", 21), ("decode64", 0)])
def test_w4a8_full_size_whole_groups(name, layer):
    import os
    oracle.set_threads(max(1, min(16, len(os.sched_getaffinity(0)))))
    case = Case(name, layer=layer, fmt="fp4", w4a8=True)
    case.run()
    ref = case.oracle_routing()
    assert_routing_equal(case.gpu_routing(), ref)
    counts = np.diff(ref["offsets"])[:case.E]
    nz = np.flatnonzero(counts)
    order = nz[np.argsort(counts[nz], kind="stable")]
    worst = _w4a8_groups(case, ref, [case.E, int(order[-1]), int(order[0])])
    say("  %s W4A8: max group rel err %.2e" % (name, worst))


def _fp8_weights(N, K, seed=0):
    wc, ws = synth.fp8_block_weights(seed, 0, N, K)
    packed = torch.empty(N * K, dtype=torch.uint8, device="cuda")
    moe.moe_fp8_prepack(N, K, torch.from_numpy(wc.reshape(-1).copy()).cuda(), packed)
    return wc, ws, packed, torch.from_numpy(ws.copy()).cuda()


def test_fp8_prepack_is_the_documented_layout():
    N, K = 48, 384
    rng = np.random.default_rng(3)
    wc = rng.integers(0, 256, (N, K), dtype=np.uint8)
    packed = torch.empty(N * K, dtype=torch.uint8, device="cuda")
    moe.moe_fp8_prepack(N, K, torch.from_numpy(wc.reshape(-1).copy()).cuda(), packed)
    got = packed.cpu().numpy()
    want = np.empty(N * K, np.uint8)
    for nt in range(N // 16):
        for kg in range(K // 128):
            blk = (nt * (K // 128) + kg) * 2048
            for l in range(64):
                n, q = 16 * nt + l % 16, l // 16
                for h in range(2):
                    want[blk + 1024 * h + 16 * l: blk + 1024 * h + 16 * l + 16] = \
                        wc[n, 128 * kg + 64 * h + 16 * q: 128 * kg + 64 * h + 16 * q + 16]
    assert np.array_equal(got, want)


def _fp8_gemm(x, N, K, packed, ws_d):
    M = x.shape[0]
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M, K // 128), dtype=torch.uint8, device="cuda")
    out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_act_quant_fp8(M, K, to_dev_bf16(x), xq, xs)
    moe.moe_fp8_block_gemm(M, N, K, xq, xs, packed, ws_d, out)
    torch.cuda.synchronize()
    return bf16_to_np_bits(out)


@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (37, 512, 384), (300, 1024, 4096), (130, 256, 1024)])
def test_fp8_block_gemm_every_element(M, N, K):
    x = synth.make_x(M, K, M + N)
    wc, ws, packed, ws_d = _fp8_weights(N, K)
    got = _fp8_gemm(x, N, K, packed, ws_d)
    ref = oracle.fp8_block_gemm(x, wc, ws)
    g, r = bits_to_f64(got), bits_to_f64(ref)
    ulps = np.abs(got.astype(np.int64) - ref.astype(np.int64))
    e = rel_err(got, ref)
    say("  fp8 block GEMM %dx%dx%d: rel err %.2e, %.4f%% of outputs one bf16 ulp off, max %d ulp" %
        (M, N, K, e, 100.0 * (ulps == 1).mean(), ulps.max()))
    assert e <= TOL


def test_fp8_block_gemm_full_size_sampled_rows():
    # an 8192-token prefill through a 4096 x 4096 projection; the oracle
    # computes three rows
    M, N, K = 8192, 4096, 4096
    x = synth.make_x(M, K, 23)
    wc, ws, packed, ws_d = _fp8_weights(N, K, seed=1)
    got = _fp8_gemm(x, N, K, packed, ws_d)
    rows = [0, 4097, 8191]
    ref = oracle.fp8_block_gemm(x[rows], wc, ws)
    e = rel_err(got[rows], ref)
    say("  fp8 block GEMM 8192x4096x4096, rows %s: rel err %.2e" % (rows, e))
    assert e <= TOL
