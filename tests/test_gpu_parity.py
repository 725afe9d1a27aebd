"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Routing (logits, expert indices, weights) and the permutation must be
bit-identical; layer outputs within 2e-2 * max|ref| (bf16 activations, fp32
accumulation).  Small shapes compare every output element; the full-size
workloads compare all routing and sampled tokens' outputs, which the oracle
computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_routed_expert_moe_amd as moe
from gpu_common import (TOL, Case, assert_routing_equal, bf16_to_np_bits, rel_err, say,
                        to_dev_bf16)

pytestmark = pytest.mark.gpu


def test_device_generator_matches_host_generator():
    say("device generator twin")
    for (layer, g0, ng, N, K) in [(0, 0, 3, 512, 512), (5, 100, 1, 4096, 4096), (42, 256, 1, 4096, 2048)]:
        codes = torch.empty(ng * N * K // 2, dtype=torch.uint8, device="cuda")
        scales = torch.empty(ng * N * (K // 128), dtype=torch.float16, device="cuda")
        for kind, skind in ((synth.KIND_W13, synth.KIND_S13), (synth.KIND_W2, synth.KIND_S2)):
            moe.moe_gen_int4_codes(0, layer, g0, ng, kind, N, K, codes)
            moe.moe_gen_fp16_scales(0, layer, g0, ng, skind, N, K, scales)
            torch.cuda.synchronize()
            dc = codes.cpu().numpy().reshape(ng, N, K // 2)
            ds = scales.cpu().numpy().reshape(ng, N, K // 128)
            for i in range(ng):
                assert np.array_equal(dc[i], synth.int4_codes(0, layer, g0 + i, kind, N, K))
                assert np.array_equal(ds[i].view(np.uint16),
                                      synth.fp16_scales(0, layer, g0 + i, skind, N, K).view(np.uint16))


def _host_prepack(canon: np.ndarray, G: int, N: int, K: int) -> np.ndarray:
    """The streamed layout as the header defines it, built with numpy."""
    c = canon.reshape(G, N, K // 2)
    lo, hi = c & 0xF, c >> 4
    codes = np.empty((G, N, K), np.uint32)
    codes[:, :, 0::2], codes[:, :, 1::2] = lo, hi
    codes ^= 8                                               # offset binary
    # [G][N/16][16 rows][K/128][4 quarters][4 words][8 elements]
    v = codes.reshape(G, N // 16, 16, K // 128, 4, 4, 8)
    word = np.zeros(v.shape[:-1], np.uint32)
    for j in range(4):
        word |= v[..., 2 * j] << (4 * j)
        word |= v[..., 2 * j + 1] << (16 + 4 * j)
    # lane = row + 16*quarter; block order (g, nt, kg, lane, word)
    word = word.transpose(0, 1, 3, 4, 2, 5)                  # G, NT, KG, quarter, row, word
    return word.reshape(-1).astype("<u4").view(np.uint8)


def test_prepack_is_the_documented_permutation():
    say("prepack layout")
    rng = np.random.default_rng(0)
    for G, N, K in [(2, 64, 256), (1, 4096, 2048)]:
        canon = rng.integers(0, 256, G * N * K // 2, dtype=np.uint8)
        got = moe.prepack(torch.from_numpy(canon).cuda(), G, N, K).cpu().numpy()
        assert np.array_equal(got, _host_prepack(canon, G, N, K))


def _full_oracle(case: Case):
    w13, s13, w2, s2 = case.stacked_weights()
    return oracle.layer_forward(case.x, case.wr, case.bias, w13, s13, w2, s2, k=case.k,
                                n_shared=case.ns, routed_scale=case.routed_scale, fmt=case.fmt)


def _check_full(case: Case):
    out = bf16_to_np_bits(case.run())
    ref = _full_oracle(case)
    assert_routing_equal(case.gpu_routing(), ref)
    h = bf16_to_np_bits(case.buf.h)
    eh, eo = rel_err(h, ref["h"]), rel_err(out, ref["out"])
    lay = case.layer_obj
    if lay.one_launch(case.T) or lay.fused_down(case.T):  # these paths never store y
        say("  rel err h %.2e out %.2e" % (eh, eo))
    else:
        ey = rel_err(bf16_to_np_bits(case.buf.y), ref["y"])
        say("  rel err h %.2e y %.2e out %.2e" % (eh, ey, eo))
        assert ey <= TOL
    assert eh <= TOL and eo <= TOL


def test_tiny_layer_every_element():
    _check_full(Case("tiny"))


@pytest.mark.parametrize("shape", [
    dict(T=37, H=1024, E=40, k=3, I=384, n_shared=1),   # ragged groups, E < 256
    dict(T=5, H=512, E=8, k=8, I=128, n_shared=0),      # k = E = 8, no shared expert
    dict(T=130, H=512, E=16, k=2, I=256, n_shared=1),   # several 16-row tiles per group
    dict(T=1, H=2048, E=64, k=4, I=256, n_shared=1),
    dict(T=300, H=512, E=256, k=6, I=128, n_shared=1),  # many near-empty groups (weight stream)
    dict(T=420, H=512, E=256, k=6, I=128, n_shared=1),  # the same on the tiled kernel
])
def test_ragged_and_edge_shapes_every_element(shape):
    _check_full(Case("shape", seed=7, weights="host", **shape))


@pytest.mark.parametrize("shape", [
    dict(T=400, H=4096, E=8, k=2, I=2048, n_shared=1),   # ~100-row groups, a 400-row shared group
    dict(T=384, H=4096, E=32, k=4, I=2048, n_shared=0),  # ~48-row groups, no shared expert
    dict(T=512, H=2048, E=16, k=3, I=4096, n_shared=1),  # gate/up K = 2048, down K = 4096
])
def test_tiled_full_k_every_element(shape):
    # the tiled kernel at the layer's K of 2048 and 4096 (32 and 16 k groups:
    # the steady state and tail of its k pipeline at full depth): every
    # element of h, y and the output against the oracle, ragged groups
    import os
    oracle.set_threads(max(1, min(16, len(os.sched_getaffinity(0)))))
    _check_full(Case("shape", seed=11, weights="host", **shape))


def test_routed_scale_and_one_expert_identity():
    # every token to expert 5 (bias +10), k = 1, no shared expert: the layer is
    # expert 5's dense MLP, scaled by routed_scale
    case = Case("one-expert", T=24, H=512, E=16, k=1, I=256, n_shared=0, seed=3, weights="host",
                routed_scale=1.0)
    case.bias[:] = 0
    case.bias[5] = 10.0
    case.layer_obj.gate_bias.copy_(torch.from_numpy(case.bias))
    _check_full(case)
    assert np.all(case.buf.topk_idx.cpu().numpy() == 5)


def _sampled(case: Case, tokens):
    out = bf16_to_np_bits(case.run())
    ref = case.oracle_routing()
    assert_routing_equal(case.gpu_routing(), ref)
    got = out[tokens]
    exp = case.oracle_tokens(tokens, ref)
    e = rel_err(got, exp)
    say("  sampled tokens %s rel err %.2e" % (list(tokens), e))
    assert e <= TOL
    return ref


def test_decode_bs1_full_size():
    _sampled(Case("decode1"), [0])


def test_decode_bs64_zipf_full_size():
    case = Case("decode64")
    ref = _sampled(case, [0, 17, 63])
    counts = np.diff(ref["offsets"])[:-1]
    hot = int(np.argmax(counts))
    say("  realised load: %d distinct experts, hottest %d rows" % ((counts > 0).sum(), counts.max()))
    assert counts.max() >= 16  # the skew spans several 16-row tiles
    hot_tokens = [t for t in range(case.T) if hot in ref["idx"][t]][:2]
    out = bf16_to_np_bits(case.buf.out)
    assert rel_err(out[hot_tokens], case.oracle_tokens(hot_tokens, ref)) <= TOL


def test_prefill_8192_full_size():
    _sampled(Case("prefill8k"), [0, 4097, 8191])


@pytest.mark.parametrize("layer", [0, 42])
def test_stack_layer_full_size(layer):
    _sampled(Case("stack43", layer=layer), [1, 2047])


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5])
def test_fused_route_permute_small_batches(T):
    # one launch for T <= 4 (last router workgroup selects and sorts), the
    # separate kernels above; the counter must come back to zero every call
    case = Case("decode1", T=T, seed=11)
    for _ in range(3):
        case.run()
        assert_routing_equal(case.gpu_routing(), case.oracle_routing())
        assert int(case.buf.ws[:4].view(torch.int32).item()) == 0
    tiny = Case("tiny", T=T, seed=12, E=16, k=2, weights="host")
    tiny.run()
    assert_routing_equal(tiny.gpu_routing(), tiny.oracle_routing())
    assert int(tiny.buf.ws[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("T,H,E", [
    (77, 4096, 40),    # sixteen experts per workgroup: a ragged token block and an expert block of 8
    (65, 2048, 256),   # H/512 = 4, just past four experts per workgroup
    (64, 4096, 256),   # four experts per workgroup
    (1030, 512, 24),   # H/512 = 1
    # from 512 tokens the 16 x 16 block kernel: whole blocks at the layer's
    # width, ragged token and expert blocks, every H/512
    (512, 4096, 256),
    (530, 2048, 40),
    (1000, 4096, 256),
    (600, 1024, 20),
])
def test_router_logits_bit_exact(T, H, E):
    say("router T=%d H=%d E=%d" % (T, H, E))
    case = Case("shape", T=T, H=H, E=E, k=6, I=128, n_shared=1, seed=13, weights="host")
    case.run()
    assert_routing_equal(case.gpu_routing(), case.oracle_routing())


@pytest.mark.parametrize("T,one_launch", [(1, True), (1, False), (5, False), (300, False)])
def test_routing_ties_go_to_the_lower_index(T, one_launch):
    # equal router rows and gate biases give bit-equal keys: experts 4i..4i+3
    # (the four keys one lane of the selecting wave holds) copy expert 4i,
    # then experts 1, 22 and 43 (in other lanes) copy expert 60.  Raised
    # biases put the tied keys at the top, so the choice and its slot order
    # turn on the tie rule: equal keys go to the lower index first.
    case = Case("ties", T=T, H=2048, E=64, k=6, I=256, n_shared=1, seed=5, weights="host")
    for e in range(case.E):
        case.wr[e] = case.wr[4 * (e // 4)]
        case.bias[e] = case.bias[4 * (e // 4)]
    for e in (1, 22, 43):
        case.wr[e] = case.wr[60]
        case.bias[e] = case.bias[60]
    case.bias[[1, 22, 43, 60]] = 0.5
    case.bias[8:12] = 0.45
    case.layer_obj.w_router = to_dev_bf16(case.wr)
    case.layer_obj.gate_bias = torch.from_numpy(case.bias).cuda()
    case.layer_obj.fuse_token = one_launch
    assert case.layer_obj.one_launch(T) == one_launch
    ref = case.oracle_routing()
    tied = sum(int(np.isin(ref["idx"][t], [1, 22, 43, 60]).sum() >= 2) for t in range(T))
    say("  tokens with at least two of the four tied experts chosen: %d of %d" % (tied, T))
    assert tied >= (T + 1) // 2
    for _ in range(2):
        case.run()
        assert_routing_equal(case.gpu_routing(), ref)


def test_outputs_are_deterministic():
    case = Case("decode64", seed=1)
    a = bf16_to_np_bits(case.run()).copy()
    h1 = bf16_to_np_bits(case.buf.h).copy()
    b = bf16_to_np_bits(case.run())
    assert np.array_equal(a, b)
    assert np.array_equal(h1, bf16_to_np_bits(case.buf.h))


def test_zero_tokens_is_a_no_op():
    say("T = 0")
    d = moe.MoeLayerDesc.make(4096, 2048, 256, 6)
    e = torch.empty(0, device="cuda")
    lib = moe._lib.lib()
    import ctypes
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.moe_route(ctypes.byref(d), 0, None, None, None, None, None, None, s) == 0
    assert lib.moe_permute(ctypes.byref(d), 0, None, None, None, None, None, 0, s) == 0
    assert lib.moe_route_permute(ctypes.byref(d), 0, None, None, None, None, None, None, None, None, None,
                                 None, 0, s) == 0
    assert lib.moe_combine(ctypes.byref(d), 0, None, None, None, None, s) == 0
    assert lib.moe_w4a16_grouped_gemm(ctypes.byref(d), 0, None, None, 0, None, 4096, 2048, None, None,
                                      None, 0, None, s) == 0
    assert lib.moe_row_sums(0, 4096, None, None, s) == 0
    torch.cuda.synchronize()
    del e


@pytest.mark.parametrize("T,E,k,ns", [
    (5, 256, 6, 1), (1023, 256, 6, 1), (1024, 256, 6, 1), (1025, 256, 6, 1),  # one chunk of 1024 tokens, then two
    (3000, 16, 8, 0), (8192, 256, 6, 1), (2049, 1, 1, 1),                   # no shared expert; one group takes all
])
def test_permute_across_token_chunks(T, E, k, ns):
    # each workgroup sorts one 1024-token chunk and counts every chunk before
    # its own: the permutation must still be the oracle's stable counting sort
    say("permute T=%d E=%d k=%d ns=%d" % (T, E, k, ns))
    rng = np.random.default_rng(T + E)
    p = rng.zipf(1.3, size=E).astype(np.float64)  # skewed loads: some groups span several chunks densely
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    d = moe.MoeLayerDesc.make(512, 256, E, k, n_shared=ns)
    G, R = E + ns, T * (k + ns)
    off = torch.full((G + 1,), -7, dtype=torch.int32, device="cuda")
    st = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    ros = torch.full((T * (k + ns),), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((moe.moe_workspace_bytes(d, T),), 0x5A, dtype=torch.uint8, device="cuda")
    moe.moe_permute(d, T, torch.from_numpy(idx).cuda(), off, st, ros, ws=ws)
    torch.cuda.synchronize()
    r_off, r_st, r_ros = oracle.permute(idx, E, ns)
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(st.cpu().numpy(), r_st)
    assert np.array_equal(ros.cpu().numpy().reshape(r_ros.shape), r_ros)


def test_row_sums_match_fp64_within_fp32_bound():
    say("row sums")
    rng = np.random.default_rng(5)
    for rows, K in [(1, 128), (37, 384), (300, 4096), (5, 2048)]:
        a = synth.f32_to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
        sums = torch.empty((rows, K // 128), dtype=torch.float32, device="cuda")
        moe.moe_row_sums(rows, K, to_dev_bf16(a), sums)
        got = sums.cpu().numpy().astype(np.float64)
        af = synth.bf16_bits_to_f32(a).astype(np.float64).reshape(rows, K // 128, 128)
        ref = af.sum(axis=2)
        bound = 8 * 2.0 ** -24 * np.abs(af).sum(axis=2)  # 7 adds in a lane + 4 pairwise levels
        assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("shape", [
    dict(T=400, E=16, k=2),   # ~71 rows per group: 64-row tiles
    dict(T=512, E=4, k=2),    # ~300 rows per group: 128-row tiles
])
def test_tiled_gemm_with_and_without_row_sums(shape):
    # from MOE_TILED_MIN_TOKENS on, the offset correction comes from the row
    # sums when given and from the matrix cores otherwise: both within the
    # tolerance of the oracle, and within fp32 rounding of each other
    case = Case("shape", H=512, I=256, n_shared=1, seed=9, weights="host", **shape)
    ref = _full_oracle(case)
    case.run()
    d, T, b, lay = case.desc, case.T, case.buf, case.layer_obj
    h_sums = bf16_to_np_bits(b.h).copy()
    ex = lay.experts
    moe.moe_w4a16_grouped_gemm(d, T, case.xd, b.sorted_token, T, None, 2 * case.I, case.H, ex.w13,
                               ex.s13, b.group_offsets, moe.MOE_ACT_SWIGLU, b.h)
    torch.cuda.synchronize()
    h_mfma = bf16_to_np_bits(b.h)
    e1, e2 = rel_err(h_sums, ref["h"]), rel_err(h_mfma, ref["h"])
    say("  h rel err with sums %.2e, without %.2e" % (e1, e2))
    assert e1 <= TOL and e2 <= TOL
    diff = np.abs(synth.bf16_bits_to_f32(h_sums) - synth.bf16_bits_to_f32(h_mfma))
    assert diff.max() <= 2.0 ** -7 * np.abs(synth.bf16_bits_to_f32(h_mfma)).max()  # one bf16 ulp


@pytest.mark.parametrize("shape", [
    dict(T=400, E=16, k=2),   # 64-row tiles
    dict(T=512, E=4, k=2),    # 128-row tiles
])
def test_tiled_gemm_scales_two_byte_aligned(shape):
    # the tile's fp16 scales go into LDS by direct loads when the scale array
    # is 4-byte aligned and through registers when it is only 2-byte aligned
    # (all the ABI asks): the same h bit for bit
    case = Case("shape", H=512, I=256, n_shared=1, seed=9, weights="host", **shape)
    case.run()
    d, T, b, ex = case.desc, case.T, case.buf, case.layer_obj.experts
    assert ex.s13.data_ptr() % 4 == 0
    moe.moe_w4a16_grouped_gemm(d, T, case.xd, b.sorted_token, T, None, 2 * case.I, case.H, ex.w13,
                               ex.s13, b.group_offsets, moe.MOE_ACT_SWIGLU, b.h)
    torch.cuda.synchronize()
    h_aligned = bf16_to_np_bits(b.h).copy()
    spare = torch.empty(ex.s13.numel() + 1, dtype=torch.float16, device=ex.s13.device)
    s_odd = spare[1:]
    s_odd.copy_(ex.s13.reshape(-1))
    assert s_odd.data_ptr() % 4 == 2
    b.h.zero_()
    moe.moe_w4a16_grouped_gemm(d, T, case.xd, b.sorted_token, T, None, 2 * case.I, case.H, ex.w13,
                               s_odd, b.group_offsets, moe.MOE_ACT_SWIGLU, b.h)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_np_bits(b.h), h_aligned)


@pytest.mark.parametrize("shape", [
    dict(T=1, H=4096, E=256, k=6, I=2048, n_shared=1),   # the decode workload's shape
    dict(T=3, H=1024, E=40, k=3, I=512, n_shared=1),     # K/128 = 4
    dict(T=4, H=512, E=16, k=8, I=1024, n_shared=0),     # K/128 = 8, no shared expert
    dict(T=2, H=512, E=8, k=2, I=4096, n_shared=1),      # K/128 = 32
])
def test_fused_down_combine_matches_oracle_and_unfused_path(shape):
    case = Case("shape", seed=13, weights="host", **shape)
    case.layer_obj.fuse_token = False  # the one-launch decode step is tested below
    assert case.layer_obj.fused_down(case.T)
    fused = bf16_to_np_bits(case.run()).copy()
    ref = _full_oracle(case)
    assert_routing_equal(case.gpu_routing(), ref)
    e1 = rel_err(fused, ref["out"])
    case.layer_obj.fuse_decode = False
    unfused = bf16_to_np_bits(case.run()).copy()
    e2 = rel_err(unfused, ref["out"])
    say("  out rel err fused %.2e, down GEMM + combine %.2e" % (e1, e2))
    assert e1 <= TOL and e2 <= TOL
    a, b = synth.bf16_bits_to_f32(fused), synth.bf16_bits_to_f32(unfused)
    assert np.abs(a - b).max() <= 2e-2 * np.abs(b).max()


def _decode_token_case(shape, seed, weights, routed_scale=1.0):
    case = Case("shape", T=1, seed=seed, weights=weights, routed_scale=routed_scale, **shape)
    assert case.layer_obj.one_launch(1), "the device does not support this decode shape"
    return case


def _run_decode_token_three_times(case: Case):
    # three calls in a row: no wait timed out (error word 3), the epoch (word
    # 4) advances once per call, and the results repeat bit for bit
    outs = []
    e0 = int(case.buf.decode_ws[4].item())
    for i in range(3):
        outs.append(bf16_to_np_bits(case.run()).copy())
        ws = case.buf.decode_ws[:5].cpu().numpy()
        assert ws[3] == 0, "a wait timed out"
        assert ws[4] == e0 + i + 1, "epoch %d after call %d" % (ws[4], i)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    return outs[0]


@pytest.mark.parametrize("shape", [
    dict(H=2048, E=64, k=4, I=256, n_shared=1),     # E < 256: most workgroups compute no logit
    dict(H=2048, E=16, k=8, I=1024, n_shared=0),    # no shared expert, two tiles per workgroup
    dict(H=2048, E=128, k=6, I=1536, n_shared=1),   # I/128 = 12, three tiles per workgroup
    dict(H=4096, E=32, k=2, I=512, n_shared=1),     # K/128 = 32 with few tiles
])
def test_decode_token_every_element(shape):
    case = _decode_token_case(shape, seed=21, weights="host")
    out = _run_decode_token_three_times(case)
    ref = _full_oracle(case)
    assert_routing_equal(case.gpu_routing(), ref)
    h = bf16_to_np_bits(case.buf.h)
    eh, eo = rel_err(h, ref["h"]), rel_err(out, ref["out"])
    # the same layer through the separate launches
    case.layer_obj.fuse_token = False
    sep = bf16_to_np_bits(case.run()).copy()
    a, b = synth.bf16_bits_to_f32(out), synth.bf16_bits_to_f32(sep)
    say("  rel err h %.2e out %.2e; vs separate launches %.2e" %
        (eh, eo, np.abs(a - b).max() / np.abs(b).max()))
    assert eh <= TOL and eo <= TOL
    assert np.abs(a - b).max() <= 2e-2 * np.abs(b).max()


@pytest.mark.parametrize("seed,routed_scale", [(0, 1.0), (31, 2.5)])
def test_decode_token_full_size(seed, routed_scale):
    # the decode workload's shape (H 4096, 256 experts top-6 + shared, I 2048)
    case = _decode_token_case(dict(H=4096, E=256, k=6, I=2048, n_shared=1), seed=seed,
                              weights="device", routed_scale=routed_scale)
    out = _run_decode_token_three_times(case)
    ref = case.oracle_routing()
    assert_routing_equal(case.gpu_routing(), ref)
    h_fused = bf16_to_np_bits(case.buf.h).copy()
    e = rel_err(out, case.oracle_tokens([0], ref))
    case.layer_obj.fuse_token = False
    sep = bf16_to_np_bits(case.run()).copy()
    h_sep = bf16_to_np_bits(case.buf.h)
    eh = rel_err(h_fused, h_sep)
    say("  out rel err %.2e; h vs separate launches %.2e" % (e, eh))
    assert e <= TOL and eh <= TOL
    assert rel_err(out, sep) <= TOL


def test_decode_token_alternating_layers_share_a_workspace():
    # the benchmark's pattern: consecutive calls on different layers with one
    # buffer set; each call's routing still matches the oracle
    cases = [_decode_token_case(dict(H=2048, E=64, k=6, I=512, n_shared=1), seed=s, weights="host")
             for s in (40, 41)]
    buf = cases[0].buf
    for c in cases:
        c.buf = buf
    for rep in range(2):
        for c in cases:
            c.run()
            assert_routing_equal(c.gpu_routing(), c.oracle_routing())
            assert int(buf.decode_ws[3].item()) == 0


def test_decode_token_error_word_is_sticky_until_the_workspace_is_zeroed():
    # the state a timed-out wait leaves (word 3 raised), forced from the host:
    # the next call returns at once, writes nothing and does not advance the
    # epoch; check_decode raises and zeroes the workspace; the call after that
    # is correct again
    case = _decode_token_case(dict(H=2048, E=64, k=4, I=256, n_shared=1), seed=23, weights="host")
    good = bf16_to_np_bits(case.run()).copy()
    case.buf.check_decode()
    ws = case.buf.decode_ws
    epoch = int(ws[4].item())
    ws[3] = 1
    case.buf.out.zero_()
    case.buf.topk_idx.fill_(-5)
    case.run()
    assert int(ws[4].item()) == epoch, "the epoch advanced after an error"
    assert np.all(case.buf.topk_idx.cpu().numpy() == -5), "a call after an error wrote its routing"
    assert not np.any(bf16_to_np_bits(case.buf.out)), "a call after an error wrote its output"
    with pytest.raises(moe.DecodeTimeout):
        case.buf.check_decode()
    assert int(ws.abs().sum().item()) == 0
    again = bf16_to_np_bits(case.run()).copy()
    case.buf.check_decode()
    assert_routing_equal(case.gpu_routing(), case.oracle_routing())
    assert np.array_equal(good, again)
    say("  sticky error word: call skipped, raised once, clean after the reset")
