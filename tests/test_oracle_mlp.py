"""Pins of the oracle's expert MLP, combine and whole-layer assembly.

Readings (pages silent): SwiGLU on the gate/up pair, W13 rows [0,I) = gate,
[I,2I) = up; h and y rounded to bf16 (the "A16"); shared expert added with
weight 1.  Pins: worked examples whose values are derived by hand in the
comments, layer identities that reduce to a dense MLP (every routed expert
identical; every token routed to one expert, the identity named for this
layer), x = 0, exact doubling, and an fp64 numpy cross-check with an
independent INT4 decode.
"""
import math

import numpy as np
import pytest

import oracle
import synth

BF16_ONE = 0x3F80


def _const_codes(n, k, code):
    nib = code & 0xF
    return np.full((n, k // 2), nib | (nib << 4), np.uint8)


def _const_scales(n, k, value):
    return np.full((n, k // 128), value, np.float16)


def _one_expert_layer(gate_code, up_code, down_code, H=512, I=128):
    w13 = np.concatenate([_const_codes(I, H, gate_code), _const_codes(I, H, up_code)])[None]
    s13 = np.concatenate([_const_scales(I, H, 2.0 ** -10), _const_scales(I, H, 2.0 ** -9)])[None]
    w2 = _const_codes(H, I, down_code)[None]
    s2 = _const_scales(H, I, 2.0 ** -4)[None]
    return w13, s13, w2, s2


def _run_one_expert(gate_code, up_code, down_code, n_shared=0):
    H, I = 512, 128
    w13, s13, w2, s2 = _one_expert_layer(gate_code, up_code, down_code, H, I)
    if n_shared:
        w13, s13, w2, s2 = [np.concatenate([a, a]) for a in (w13, s13, w2, s2)]
    x = np.full((3, H), BF16_ONE, np.uint16)
    wr = synth.make_router(1, H, seed=1)
    bias = np.zeros(1, np.float32)
    return oracle.layer_forward(x, wr, bias, w13, s13, w2, s2, k=1, n_shared=n_shared)


def test_worked_example_positive_gate():
    # x = 1 everywhere (H = 512).  Gate codes +2, scale 2^-10: G = 512*2*2^-10 = 1.
    # Up codes +4, scale 2^-9: U = 512*4*2^-9 = 4.
    # a = 4*sigmoid(1) = 2.92423431...; bf16 keeps 8 bits: 187.15/128*2 -> h = 2.921875.
    # Down codes -1, scale 2^-4: y = 128 * 2.921875 * (-1/16) = -23.375 (8 bits, exact).
    # One expert, k = 1: weight s/s = 1, so out = -23.375.
    o = _run_one_expert(2, 4, -1)
    h = synth.bf16_bits_to_f32(o["h"])
    out = synth.bf16_bits_to_f32(o["out"])
    assert np.all(h == 2.921875)
    assert np.all(out == -23.375)
    assert np.all(o["w"] == 1.0)
    # gate and up swapped gives silu(4)*1 = 3.928..., a different h
    o2 = _run_one_expert(4, 2, -1)
    assert not np.any(synth.bf16_bits_to_f32(o2["h"]) == 2.921875)


def test_worked_example_negative_gate():
    # Gate codes -2: G = -1, a = -4*sigmoid(-1) = -1.07576568...; 137.698 -> 138:
    # h = -138/128 = -1.078125.  y = 128 * -1.078125 * (-1/16) = 8.625.
    o = _run_one_expert(-2, 4, -1)
    assert np.all(synth.bf16_bits_to_f32(o["h"]) == -1.078125)
    assert np.all(synth.bf16_bits_to_f32(o["out"]) == 8.625)


def test_worked_example_shared_expert_adds_with_weight_one():
    # shared expert identical to the routed one: out = bf16(-23.375 + -23.375)
    o = _run_one_expert(2, 4, -1, n_shared=1)
    assert np.all(synth.bf16_bits_to_f32(o["out"]) == -46.75)
    assert list(o["offsets"]) == [0, 3, 6]


def _decode_codes(w):
    codes = np.empty((w.shape[0], w.shape[1] * 2), np.int64)
    codes[:, 0::2] = (w.astype(np.int16) << 12).astype(np.int16) >> 12
    codes[:, 1::2] = w.astype(np.int8) >> 4
    return codes


def _bf16(a):
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


def _within_one_bf16_ulp(out, ref):
    """|out - ref| <= one bf16 ulp of ref (2^-7 relative) plus a tiny absolute slack."""
    return np.all(np.abs(out - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6 * np.max(np.abs(ref)))


def _dense_ref(x_bits, w13, s13, w2, s2):
    """Textbook SwiGLU MLP in fp64 with bf16 h and y, independent INT4 decode."""
    I = w2.shape[1] * 2
    X = synth.bf16_bits_to_f32(x_bits).astype(np.float64)
    W13 = _decode_codes(w13) * np.repeat(s13.astype(np.float64), 128, axis=1)
    W2 = _decode_codes(w2) * np.repeat(s2.astype(np.float64), 128, axis=1)
    gu = X @ W13.T
    g, u = gu[:, :I], gu[:, I:]
    h = g / (1.0 + np.exp(-g)) * u
    return _bf16(_bf16(h) @ W2.T)


def _tiny_weights(seed, G, H=512, I=256):
    return synth.stacked_expert_weights(seed, 0, G, H, I)


def test_all_routed_experts_identical_reduces_to_dense():
    T, H, I, E, k = 8, 512, 256, 16, 2
    w13, s13, w2, s2 = _tiny_weights(0, E + 1, H, I)
    for a in (w13, s13, w2, s2):
        a[1:E] = a[0]
    x, wr, bias = synth.make_router_inputs("tiny")
    o = oracle.layer_forward(x, wr, bias, w13, s13, w2, s2, k=k, n_shared=1)
    yr = _dense_ref(x, w13[0], s13[0], w2[0], s2[0])
    ys = _dense_ref(x, w13[E], s13[E], w2[E], s2[E])
    ref = _bf16(yr + ys)   # the two routed weights sum to 1 within 2^-23
    out = synth.bf16_bits_to_f32(o["out"]).astype(np.float64)
    assert _within_one_bf16_ulp(out, ref)


def test_every_token_to_one_expert_equals_its_dense_mlp():
    T, H, I, E = 8, 512, 256, 16
    w13, s13, w2, s2 = _tiny_weights(1, E + 1, H, I)
    x, wr, _ = synth.make_router_inputs("tiny")
    bias = np.zeros(E, np.float32)
    bias[7] = 10.0
    o = oracle.layer_forward(x, wr, bias, w13[:E], s13[:E], w2[:E], s2[:E], k=1, n_shared=0)
    assert np.all(o["idx"] == 7) and np.all(o["w"] == 1.0)
    ref = _dense_ref(x, w13[7], s13[7], w2[7], s2[7])
    out = synth.bf16_bits_to_f32(o["out"]).astype(np.float64)
    assert _within_one_bf16_ulp(out, ref)
    # routed rows equal the expert's own y
    assert np.array_equal(o["out"], o["y"][o["row_of_slot"][:, 0]])


def test_zero_input_gives_zero_output():
    w13, s13, w2, s2 = _tiny_weights(2, 17)
    _, wr, bias = synth.make_router_inputs("tiny")
    x = np.zeros((8, 512), np.uint16)
    o = oracle.layer_forward(x, wr, bias, w13, s13, w2, s2, k=2, n_shared=1)
    assert np.all(synth.bf16_bits_to_f32(o["out"]) == 0.0)


def test_doubling_down_scales_doubles_output_exactly():
    w13, s13, w2, s2 = _tiny_weights(3, 17)
    x, wr, bias = synth.make_router_inputs("tiny")
    o1 = oracle.layer_forward(x, wr, bias, w13, s13, w2, s2, k=2, n_shared=1)
    o2 = oracle.layer_forward(x, wr, bias, w13, s13, w2, (s2 * 2).astype(np.float16), k=2, n_shared=1)
    assert np.array_equal(synth.bf16_bits_to_f32(o2["out"]), 2 * synth.bf16_bits_to_f32(o1["out"]))


def test_layer_matches_fp64_numpy_recomputation():
    T, H, I, E, k = 8, 512, 256, 16, 2
    w13, s13, w2, s2 = _tiny_weights(0, E + 1, H, I)
    x, wr, bias = synth.make_router_inputs("tiny")
    o = oracle.layer_forward(x, wr, bias, w13, s13, w2, s2, k=k, n_shared=1)
    ref = np.zeros((T, H))
    for t in range(T):
        ref[t] = _dense_ref(x[t:t + 1], w13[E], s13[E], w2[E], s2[E])[0]
        for j in range(k):
            e = o["idx"][t, j]
            y = _dense_ref(x[t:t + 1], w13[e], s13[e], w2[e], s2[e])[0]
            ref[t] += float(o["w"][t, j]) * y
    out = synth.bf16_bits_to_f32(o["out"]).astype(np.float64)
    assert np.max(np.abs(out - ref)) <= 1e-2 * np.max(np.abs(ref))


def test_token_outputs_matches_layer_forward():
    E, k = 16, 2
    w13, s13, w2, s2 = _tiny_weights(0, E + 1)
    x, wr, bias = synth.make_router_inputs("tiny")
    o = oracle.layer_forward(x, wr, bias, w13, s13, w2, s2, k=k, n_shared=1)
    got = oracle.token_outputs([5, 0, 3], x, o["idx"], o["w"],
                               lambda g: (w13[g], s13[g], w2[g], s2[g]), E, 1)
    assert np.array_equal(got, o["out"][[5, 0, 3]])
