"""Pins of the oracle's fp8 functions: the e4m3 format, the activation
quantisation per token per 128 elements, the W4A8 expert MLP and the
FP8_BLOCK GEMM ("Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass
through the model": e4m3 activations scaled per token per 128 elements; model
card "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Component precisions":
FP8_BLOCK 128x128 with dynamic ue8m0 scales).

Each is tied to something other than the oracle: torch's float8_e4m3fn
(an independent implementation of the OCP format) for decoding and
round-to-nearest-even encoding; constants of the format; brute force over
the finite values; the already-pinned W4A16/FP4 oracle on inputs the fp8
path represents exactly; an fp64 numpy recomputation."""
import numpy as np
import pytest
import torch

import oracle
import synth

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_values_match_torch_and_the_format_constants():
    vals = np.array([oracle.e4m3_value(c) for c in range(256)])
    ref = torch_e4m3(np.arange(256))
    assert np.array_equal(np.isnan(vals), np.isnan(ref))
    assert np.array_equal(vals[FINITE], ref[FINITE])
    assert [c for c in range(256) if np.isnan(vals[c])] == [0x7F, 0xFF]   # no infinities
    assert vals[0x7E] == 448.0 and vals[0x08] == 2.0 ** -6 and vals[0x01] == 2.0 ** -9
    assert vals[0x38] == 1.0 and vals[0x80] == 0.0 and np.signbit(vals[0x80])
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)                                          # monotone
    assert np.array_equal(vals[0x80:0xFF], -pos)                             # sign symmetric
    assert np.all(np.mod(pos * 2 ** 9, 1) == 0)                              # multiples of 2^-9


def test_e4m3_encode_is_round_to_nearest_even():
    vals = np.array([oracle.e4m3_value(c) for c in FINITE])
    fin = np.array(FINITE)
    rng = np.random.default_rng(0)
    pos = np.unique(vals[vals > 0])
    mids = (pos[:-1] + pos[1:]) / 2
    xs = np.r_[mids, -mids, pos, -pos, 2.0 ** rng.uniform(-11, np.log2(448), 4000) * rng.choice([-1, 1], 4000),
               0.0, -0.0, 448.0, 1e-6]
    got = np.array([oracle.e4m3_encode(x) for x in xs])
    # torch's conversion (round to nearest, ties to even) of the same values
    want = torch.from_numpy(xs.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    # brute force: the nearest finite value, and on a tie the even code
    for x, c in zip(xs[:600], got[:600]):
        d = np.abs(vals - x)
        best = fin[d == d.min()]
        if len(best) > 1:
            best = [b for b in best if b % 2 == 0]
        assert oracle.e4m3_value(c) == oracle.e4m3_value(int(best[0]))
    assert all(oracle.e4m3_encode(oracle.e4m3_value(c)) == c for c in FINITE)  # round trip
    assert oracle.e4m3_encode(1000.0) == 0x7E and oracle.e4m3_encode(-1000.0) == 0xFE
    # NaN has one pattern per sign (S.1111.111), as torch's conversion gives
    nan_code = int(torch.tensor([float("nan")], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8))
    assert oracle.e4m3_encode(float("nan")) == nan_code == 0x7F
    assert oracle.e4m3_encode(-float("nan")) == 0xFF


def _bf16(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, np.float32))


def test_activation_scale_is_the_smallest_power_of_two_that_fits_448():
    # hand values: max|x| 448 fits scale 1; the next bf16 value (450) does not
    assert oracle.act_scale_code(_bf16([448.0, -3.0])) == 127
    assert oracle.act_scale_code(_bf16([450.0])) == 128
    assert oracle.act_scale_code(_bf16([-450.0, 1.0])) == 128
    assert oracle.act_scale_code(_bf16([1.0])) == 119        # 448 * 2^-9 < 1 <= 448 * 2^-8
    assert oracle.act_scale_code(_bf16([3.5])) == 120        # 3.5 = 448 * 2^-7 exactly
    assert oracle.act_scale_code(_bf16([0.0, -0.0])) == 127  # all zero: scale 1
    # below the UE8M0 range the scale stays at its smallest, 2^-127 (bf16
    # subnormals: max|x| < 448 * 2^-127)
    assert oracle.act_scale_code(np.array([0x0001, 0x8005, 0x007F], np.uint16)) == 0
    assert oracle.act_scale_code(_bf16([448.0 * 2.0 ** -127])) == 0
    assert oracle.act_scale_code(_bf16([480.0 * 2.0 ** -127])) == 1
    rng = np.random.default_rng(1)
    for _ in range(200):
        x = _bf16(rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 6))
        E = oracle.act_scale_code(x)
        amax = np.abs(synth.bf16_bits_to_f32(x).astype(np.float64)).max()
        assert 224.0 * 2.0 ** (E - 127) < amax <= 448.0 * 2.0 ** (E - 127)


def test_activation_quant_matches_torch_on_every_element():
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((9, 384)) * np.array([1e-3, 1, 30, 1e4, 0.5, 7, 1e-5, 2, 100])[:, None])
    x[3, 128:256] = 0                                              # a block of zeros
    codes, scales = oracle.act_quant_fp8(x)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    for r in range(x.shape[0]):
        for b in range(3):
            blk = x[r, 128 * b:128 * b + 128]
            E = scales[r, b]
            assert E == oracle.act_scale_code(blk)
            scaled = xf[r, 128 * b:128 * b + 128] * 2.0 ** (127 - int(E))
            want = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[r, 128 * b:128 * b + 128], want)
            deq = torch_e4m3(codes[r, 128 * b:128 * b + 128]) * 2.0 ** (int(E) - 127)
            assert np.all(np.abs(deq - xf[r, 128 * b:128 * b + 128]) <= 2.0 ** -4 * np.abs(xf[r, 128 * b:128 * b + 128])
                          + 2.0 ** (int(E) - 127 - 10))
    assert not np.any(codes[3, 128:256])


def _fp4_group(H, I, seed=0):
    return synth.fp4_expert_weights(seed, 3, 1, H, I)


def test_w4a8_mlp_is_the_fp4_mlp_on_the_quantised_activations():
    # gate/up: the W4A8 MLP's h equals the pinned FP4 (A16) MLP fed with the
    # dequantised fp8 activations, which bf16 holds exactly; down: y equals an
    # fp64 numpy product of the dequantised h codes and the FP4 down weights
    H, I = 512, 256
    w13, s13, w2, s2 = _fp4_group(H, I)
    x = synth.make_x(6, H, 4)
    h, hc, hs, y = oracle.expert_mlp_w4a8(x, w13, s13, w2, s2)
    xc, xs = oracle.act_quant_fp8(x)
    xdeq = torch_e4m3(xc) * np.repeat(2.0 ** (xs.astype(np.float64) - 127), 128, axis=1)
    xdeq_bits = synth.f32_to_bf16_bits(xdeq.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(xdeq_bits).astype(np.float64), xdeq)  # exact in bf16
    h_a16, _ = oracle.expert_mlp_fp4(xdeq_bits, w13, s13, w2, s2)
    assert np.array_equal(h, h_a16)
    c2, s2q = oracle.act_quant_fp8(h)
    assert np.array_equal(hc, c2) and np.array_equal(hs, s2q)
    hdeq = torch_e4m3(hc) * np.repeat(2.0 ** (hs.astype(np.float64) - 127), 128, axis=1)
    y_ref = hdeq @ oracle.dequant_fp4(w2, s2).T
    yf = synth.bf16_bits_to_f32(y).astype(np.float64)
    assert np.all(np.abs(yf - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + 1e-30)        # bf16 rounding
    z = np.zeros_like(x)
    _, _, _, yz = oracle.expert_mlp_w4a8(z, w13, s13, w2, s2)
    assert not np.any(yz & 0x7FFF)


def test_w4a8_layer_within_the_fp8_accuracy_of_the_a16_layer():
    # the accuracy contract of the variant: the W4A8 layer against the FP4
    # layer with bf16 activations on the same weights and routing
    w = synth.WORKLOADS["tiny"]
    T, H, E, k, I = w["T"], w["H"], w["E"], w["k"], w["I"]
    x, wr, bias = synth.make_router_inputs("tiny")
    w13, s13, w2, s2 = synth.stacked_fp4_expert_weights(0, 0, E + 1, H, I)
    a = oracle.layer_forward(x, wr, bias, w13, s13, w2, s2, k=k, fmt="fp4")
    b = oracle.layer_forward_w4a8(x, wr, bias, w13, s13, w2, s2, k=k)
    for key in ("logits", "idx", "w", "offsets", "sorted_token", "row_of_slot"):
        assert np.array_equal(a[key], b[key])
    oa = synth.bf16_bits_to_f32(a["out"]).astype(np.float64)
    ob = synth.bf16_bits_to_f32(b["out"]).astype(np.float64)
    err = np.abs(oa - ob).max() / np.abs(oa).max()
    assert err <= 5e-2, err


def test_fp8_block_gemm_against_numpy():
    M, N, K = 5, 256, 384
    x = synth.make_x(M, K, 6)
    wc, ws = synth.fp8_block_weights(0, 0, N, K)
    y = oracle.fp8_block_gemm(x, wc, ws)
    xc, xs = oracle.act_quant_fp8(x)
    xd = torch_e4m3(xc) * np.repeat(2.0 ** (xs.astype(np.float64) - 127), 128, axis=1)
    wd = torch_e4m3(wc.reshape(-1)).reshape(N, K) * np.repeat(np.repeat(2.0 ** (ws.astype(np.float64) - 127), 128, 0),
                                                               128, 1)
    ref = xd @ wd.T
    yf = synth.bf16_bits_to_f32(y).astype(np.float64)
    assert np.all(np.abs(yf - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def test_fp8_block_scale_placement():
    # small integers make every product and sum exact: raising one block's
    # scale byte by one doubles exactly that block's contribution
    M, N, K = 3, 256, 256
    rng = np.random.default_rng(7)
    x = _bf16(rng.integers(-3, 4, (M, K)).astype(np.float32))
    x[:, 0] = _bf16([4.0])[0]                        # every block's scale 2^-6: 64 x is exact in e4m3
    x[:, 128] = _bf16([4.0])[0]
    one, two = oracle.e4m3_encode(1.0), oracle.e4m3_encode(-0.5)
    wc = np.where(rng.random((N, K)) < 0.5, one, two).astype(np.uint8)
    ws = np.full((2, 2), 127, np.uint8)
    y0 = synth.bf16_bits_to_f32(oracle.fp8_block_gemm(x, wc, ws)).astype(np.float64)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    wf = np.where(wc == one, 1.0, -0.5)
    assert np.array_equal(y0, xf @ wf.T)
    ws2 = ws.copy()
    ws2[1, 0] = 128                                  # rows 128..255 of W, k 0..127
    y1 = synth.bf16_bits_to_f32(oracle.fp8_block_gemm(x, wc, ws2)).astype(np.float64)
    part = xf[:, :128] @ wf[128:, :128].T
    assert np.array_equal(y1[:, :128], y0[:, :128])
    assert np.array_equal(y1[:, 128:] - y0[:, 128:], part)
