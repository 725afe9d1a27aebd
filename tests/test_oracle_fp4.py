"""Pins of the oracle's FP4 expert-weight functions (E2M1 elements, UE8M0
scales per 32 elements along K) to definitions outside the oracle: the
values rebuilt from the element's bit fields as IEEE binary32 patterns,
power-of-two scales from math.ldexp, a brute-force encode/decode round
trip, and identity with the pinned INT4 path on weights both formats hold
exactly."""
import math

import numpy as np
import pytest

import oracle
import synth


def _e2m1_as_binary32(code: int) -> float:
    # the element's fields placed into a binary32 pattern: exponent field e
    # (bias 1) becomes 127 + e - 1, the mantissa bit the top fraction bit;
    # e = 0 is the subnormal 0.m * 2^0
    sign, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    if e == 0:
        bits = (0x3F000000 if m else 0)  # 0.5 or 0
    else:
        bits = ((127 + e - 1) << 23) | (m << 22)
    v = float(np.array([bits], np.uint32).view(np.float32)[0])
    return -v if sign else v


def test_fp4_element_values_from_the_bit_fields():
    got = [oracle.fp4_value(c) for c in range(16)]
    assert got == [_e2m1_as_binary32(c) for c in range(16)]
    # invariants of the format: codes 0..7 increase strictly, c ^ 8 negates,
    # the largest magnitude is 6, and 8 is a negative zero
    assert all(got[c] < got[c + 1] for c in range(7))
    assert all(got[c ^ 8] == -got[c] for c in range(16))
    assert max(got) == 6.0 and math.copysign(1.0, got[8]) == -1.0


def test_ue8m0_is_a_power_of_two():
    for E in range(255):
        assert oracle.ue8m0(E) == math.ldexp(1.0, E - 127)
    for E in range(1, 255):  # normal binary32 numbers: the byte is the exponent field
        assert oracle.ue8m0(E) == float(np.array([E << 23], np.uint32).view(np.float32)[0])
    assert math.isnan(oracle.ue8m0(255))


def test_dequant_fp4_round_trip_by_brute_force():
    # random representable weights (an element value times its block's scale),
    # encoded by searching the 16 codes, packed in canonical order (element 2c
    # in the low nibble of byte c), must dequantise to themselves
    rng = np.random.default_rng(7)
    N, K = 5, 96
    E = rng.integers(118, 125, size=(N, K // 32)).astype(np.uint8)
    codes = rng.integers(0, 16, size=(N, K))
    vals = np.array([[oracle.fp4_value(int(codes[n, k])) * 2.0 ** (int(E[n, k // 32]) - 127)
                      for k in range(K)] for n in range(N)])
    enc = np.zeros((N, K), np.int64)
    for n in range(N):
        for k in range(K):
            s = 2.0 ** (int(E[n, k // 32]) - 127)
            hits = [c for c in range(16) if oracle.fp4_value(c) * s == vals[n, k]
                    and math.copysign(1, oracle.fp4_value(c)) == math.copysign(1, vals[n, k])]
            assert hits
            enc[n, k] = hits[0]
    packed = (enc[:, 0::2] | (enc[:, 1::2] << 4)).astype(np.uint8)
    got = oracle.dequant_fp4(packed, E)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))


def _int4_and_fp4_with_equal_values(rng, rows, cols):
    # integers both formats hold exactly: |q| in {0,1,2,3,4,6}; INT4 scale
    # 2^-6 (an fp16 number), FP4 scale byte 121 (also 2^-6)
    e2m1_of = {0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 6: 7}
    q = rng.choice([-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6], size=(rows, cols))
    i4 = q & 0xF
    f4 = np.array([[e2m1_of[abs(int(v))] | (8 if v < 0 else 0) for v in row] for row in q])
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    s16 = np.full((rows, cols // 128), 2.0 ** -6, np.float16)
    s8 = np.full((rows, cols // 32), 121, np.uint8)
    return pack(i4), s16, pack(f4), s8


def test_fp4_mlp_equals_the_int4_mlp_on_equal_weights():
    rng = np.random.default_rng(3)
    H, I, n = 256, 128, 3
    w13i, s13i, w13f, s13f = _int4_and_fp4_with_equal_values(rng, 2 * I, H)
    w2i, s2i, w2f, s2f = _int4_and_fp4_with_equal_values(rng, H, I)
    assert np.array_equal(oracle.dequant(w13i, s13i), oracle.dequant_fp4(w13f, s13f))
    x = synth.make_x(n, H, seed=4)
    hi, yi = oracle.expert_mlp(x, w13i, s13i, w2i, s2i)
    hf, yf = oracle.expert_mlp_fp4(x, w13f, s13f, w2f, s2f)
    assert np.array_equal(hi, hf) and np.array_equal(yi, yf)


def test_fp4_layer_equals_the_int4_layer_on_equal_weights():
    rng = np.random.default_rng(5)
    T, H, E, k, I = 6, 512, 8, 2, 128
    G = E + 1
    parts = [(_int4_and_fp4_with_equal_values(rng, 2 * I, H), _int4_and_fp4_with_equal_values(rng, H, I))
             for _ in range(G)]
    st = lambda i, j: np.stack([p[i][j] for p in parts])
    x = synth.make_x(T, H, seed=1)
    wr = synth.make_router(E, H, seed=1)
    b = synth.make_bias(E, seed=1)
    a = oracle.layer_forward(x, wr, b, st(0, 0), st(0, 1), st(1, 0), st(1, 1), k)
    f = oracle.layer_forward(x, wr, b, st(0, 2), st(0, 3), st(1, 2), st(1, 3), k, fmt="fp4")
    for key in ("idx", "offsets", "h", "y", "out"):
        assert np.array_equal(a[key], f[key]), key


def test_fp4_generator_covers_every_code_and_scale():
    w13, s13, w2, s2 = synth.fp4_expert_weights(0, 0, 3, 256, 128)
    assert w13.shape == (256, 128) and s13.shape == (256, 8) and s2.shape == (256, 4)
    nib = np.concatenate([w13 & 0xF, w13 >> 4]).ravel()
    assert set(np.unique(nib)) == set(range(16))
    assert set(np.unique(s13)) == {120, 121, 122, 123}
