"""Pins of the oracle's router logits (fp32, fixed lane order, then butterfly).

The pages fix no router formula; the order is this build's definition so
that a 64-lane wavefront reproduces it bit for bit.  The tests check exact
values the definition implies (worked by hand below), exactness on
integer-valued inputs, and Higham's recursive-summation bound on random
inputs.
"""
import numpy as np

import oracle
import synth


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_one_hot_input_returns_the_weight():
    H, E = 1024, 8
    wr = synth.make_router(E, H, seed=3)
    for i in (0, 7, 8, 511, 512, 1023):
        x = np.zeros((1, H), np.float32)
        x[0, i] = 1.0
        lg = oracle.router_logits(_bits(x), wr)
        assert np.array_equal(lg[0], synth.bf16_bits_to_f32(wr[:, i]))


def test_integer_inputs_sum_exactly():
    rng = np.random.default_rng(1)
    H, E, T = 2048, 5, 4
    x = rng.integers(-8, 9, (T, H)).astype(np.float32)
    w = rng.integers(-8, 9, (E, H)).astype(np.float32)
    lg = oracle.router_logits(_bits(x), _bits(w))
    assert np.array_equal(lg.astype(np.int64), x.astype(np.int64) @ w.astype(np.int64).T)


def test_summation_order_worked_example_lane_partials():
    # H = 512.  Lane l owns elements 8l..8l+7.  Products: 2^24 at element 0,
    # 1.0 at elements 1..7 (lane 0) and 1.0 at elements 8..15 (lane 1).
    # Lane 0: 2^24 + 1 rounds to 2^24 (tie to even) seven times -> 2^24.
    # Lane 1: 8.  Butterfly (d=32..1): lane 0 ends with 2^24 + 8 = 16777224.
    # The exact sum 2^24 + 15 and a single running sum (2^24) both differ.
    H = 512
    x = np.zeros((1, H), np.float32)
    w = np.zeros((1, H), np.float32)
    x[0, 0], w[0, 0] = 4096.0, 4096.0
    x[0, 1:16], w[0, 1:16] = 1.0, 1.0
    assert oracle.router_logits(_bits(x), _bits(w))[0, 0] == 16777224.0


def test_summation_order_worked_example_butterfly():
    # Lane 0 partial 1.0 (element 0), lane 1 partial 1.0 (element 8), lane 32
    # partial 2^24 (element 256).  d=32 pairs lanes 0 and 32 first:
    # 1 + 2^24 -> 2^24; lane 1 keeps 1; ...; d=1: 2^24 + 1 -> 2^24.
    # A running sum in element order would give 2^24 + 2 exactly.
    H = 512
    x = np.zeros((1, H), np.float32)
    w = np.zeros((1, H), np.float32)
    x[0, [0, 8]] = 1.0
    w[0, [0, 8]] = 1.0
    x[0, 256], w[0, 256] = 4096.0, 4096.0
    assert oracle.router_logits(_bits(x), _bits(w))[0, 0] == 16777216.0


def test_second_column_block_goes_to_the_same_lane():
    # Elements 0 and 512 both belong to lane 0 (j = 0 and j = 1); 2^24 at 0,
    # then 1.0 at 512 is absorbed; 1.0 at 8 (lane 1) survives to the end.
    H = 1024
    x = np.zeros((1, H), np.float32)
    w = np.zeros((1, H), np.float32)
    x[0, [0, 512, 8]] = [4096.0, 1.0, 1.0]
    w[0, [0, 512, 8]] = [4096.0, 1.0, 1.0]
    assert oracle.router_logits(_bits(x), _bits(w))[0, 0] == 16777216.0


def test_random_inputs_within_recursive_summation_bound():
    x, wr, _ = synth.make_router_inputs("tiny", seed=2)
    x = synth.make_x(16, 4096, seed=2)
    wr = synth.make_router(32, 4096, seed=2)
    lg = oracle.router_logits(x, wr).astype(np.float64)
    X = synth.bf16_bits_to_f32(x).astype(np.float64)
    W = synth.bf16_bits_to_f32(wr).astype(np.float64)
    exact = X @ W.T
    absum = np.abs(X) @ np.abs(W).T
    n = 4096 // 64 + 6
    bound = n * 2.0 ** -24 / (1 - n * 2.0 ** -24) * absum
    assert np.all(np.abs(lg - exact) <= bound)
