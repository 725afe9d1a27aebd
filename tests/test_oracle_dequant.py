"""Pins of the oracle's INT4 decode, fp16 decode, dequantisation and bf16 rounding.

The model card ("canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Component
precisions") fixes INT4, group_size=128, symmetric.  The nibble order and
two's-complement encoding are this build's reading; the pins below check the
oracle against independent decodings (numpy sign extension, numpy's fp16) and
hand-written values.
"""
import numpy as np

import oracle
import synth


def test_int4_code_exhaustive_against_sign_extension():
    for b in range(256):
        lo = oracle.int4_code(b, 0)
        hi = oracle.int4_code(b, 1)
        # arithmetic right shift of an int8 sign-extends the top nibble
        exp_lo = int(np.int8(np.uint8((b << 4) & 0xFF)) >> 4)
        exp_hi = int(np.int8(np.uint8(b)) >> 4)
        assert (lo, hi) == (exp_lo, exp_hi), b
    assert oracle.int4_code(0x08, 0) == -8
    assert oracle.int4_code(0x07, 0) == 7
    assert oracle.int4_code(0x0F, 0) == -1
    assert oracle.int4_code(0x80, 1) == -8
    assert oracle.int4_code(0x70, 1) == 7


def test_fp16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_f64(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(got), np.signbit(ref))  # signed zeros and NaN signs too


def test_dequant_hand_values_and_group_axis():
    # one row, K = 256: bytes hold (low, high) = (2c, 2c+1) elements
    # codes for k = 0..15: 0,1,2,3,4,5,6,7,-8,-7,...,-1 then repeated
    codes = np.array([((i % 16) - 16 if (i % 16) >= 8 else (i % 16)) for i in range(256)])
    nib = codes & 0xF
    row = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[0.5, 0.25]], dtype=np.float16)  # group 0 -> k<128, group 1 -> k>=128
    out = oracle.dequant(row, scales)
    expect = codes * np.where(np.arange(256) < 128, 0.5, 0.25)
    assert np.array_equal(out[0], expect)
    # three rows, distinct scales per (row, group): catches a transposed scale index
    w = np.repeat(row, 3, axis=0)
    s = np.array([[1, 2], [4, 8], [16, 32]], dtype=np.float16)
    out = oracle.dequant(w, s)
    for n in range(3):
        assert np.array_equal(out[n, :128], codes[:128] * float(s[n, 0]))
        assert np.array_equal(out[n, 128:], codes[128:] * float(s[n, 1]))


def test_dequant_is_exact_in_fp32_and_round_trips():
    # q*s needs at most 4+11 significant bits: exact in fp32 for every fp16 scale
    s_bits = np.arange(0x0001, 0x7C00, dtype=np.uint16)  # all finite positive fp16
    s = s_bits.view(np.float16)
    q = np.arange(-8, 8)
    prod32 = q[:, None].astype(np.float32) * s[None, :].astype(np.float32)
    prod64 = q[:, None].astype(np.float64) * s[None, :].astype(np.float64)
    assert np.array_equal(prod32.astype(np.float64), prod64)
    assert np.array_equal(np.rint(prod64 / s[None, :].astype(np.float64)), q[:, None] * np.ones_like(prod64))


def test_dequant_matches_independent_decode_on_generated_weights():
    w13, s13, _, _ = synth.expert_weights(0, 0, 3, 256, 128)
    ref_codes = np.empty((w13.shape[0], w13.shape[1] * 2), np.int64)
    ref_codes[:, 0::2] = (np.int8(0) + (w13.astype(np.int16) << 12).astype(np.int16) >> 12)
    ref_codes[:, 1::2] = w13.astype(np.int8) >> 4
    ref = ref_codes * np.repeat(s13.astype(np.float64), 128, axis=1)
    assert np.array_equal(oracle.dequant(w13, s13), ref)


def test_bf16_rounding_hand_values():
    one = 0x3F80
    assert oracle.f64_to_bf16(1.0) == one
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == one              # tie -> even (down)
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == one + 2      # tie -> even (up)
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == one + 1  # above the tie
    assert oracle.f64_to_bf16(-2.921875) == 0xC03B
    assert oracle.f64_to_bf16(3.5e38) == 0x7F80                      # overflow
    assert oracle.f64_to_bf16(2.0 ** -133) == 0x0001                 # smallest subnormal
    assert oracle.f64_to_bf16(0.0) == 0


def test_bf16_rounding_matches_fp32_path_on_fp32_values():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000)).astype(np.float32)
    ref = synth.f32_to_bf16_bits(v)
    got = np.array([oracle.f64_to_bf16(float(a)) for a in v], dtype=np.uint16)
    assert np.array_equal(got, ref)
