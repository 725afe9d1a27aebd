"""The seeded input generators: SplitMix64 against its published first outputs
and its scalar form, and the drawn tensors' ranges.  (Inputs only; no method
arithmetic lives in ``synth``.)"""
import numpy as np

import synth


def test_splitmix64_published_first_outputs_seed0():
    # first outputs of SplitMix64 (Steele, Lea & Flood 2014) seeded with 0
    assert synth.splitmix64_py(0, 0) == 0xE220A8397B1DCDAF
    assert synth.splitmix64_py(0, 1) == 0x6E789E6AA1B965F4
    assert synth.splitmix64_py(0, 2) == 0x06C45D188009454F


def test_vector_form_matches_scalar_form():
    for seed in (0, 1, 0xDEADBEEF, 2 ** 63 + 5):
        v = synth.splitmix64_block(seed, 1000, 64)
        assert [int(a) for a in v] == [synth.splitmix64_py(seed, 1000 + i) for i in range(64)]


def test_int4_codes_are_uniform_and_scales_in_range():
    w = synth.int4_codes(0, 0, 5, synth.KIND_W13, 512, 1024)
    lo = (w & 0xF).astype(np.int64)
    hi = (w >> 4).astype(np.int64)
    counts = np.bincount(np.concatenate([lo.ravel(), hi.ravel()]), minlength=16)
    assert counts.min() > 0.9 * counts.mean() and counts.max() < 1.1 * counts.mean()
    s = synth.fp16_scales(0, 0, 5, synth.KIND_S13, 512, 1024).astype(np.float64)
    assert s.min() >= 0.005 - 1e-5 and s.max() <= 0.02 + 1e-5
    assert abs(s.mean() - 0.0125) < 5e-4


def test_tensors_differ_by_layer_group_and_kind():
    a = synth.int4_codes(0, 0, 1, synth.KIND_W13, 16, 256)
    assert not np.array_equal(a, synth.int4_codes(0, 1, 1, synth.KIND_W13, 16, 256))
    assert not np.array_equal(a, synth.int4_codes(0, 0, 2, synth.KIND_W13, 16, 256))
    assert not np.array_equal(a, synth.int4_codes(0, 0, 1, synth.KIND_W2, 16, 256))
    assert np.array_equal(a, synth.int4_codes(0, 0, 1, synth.KIND_W13, 16, 256))


def test_bf16_bits_round_trip_and_rne():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0, 0.0], np.float32)
    assert list(synth.f32_to_bf16_bits(v)) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000]


def test_uniform_routing_gives_near_uniform_load():
    # the prefill workload's construction at a quarter of its tokens: every
    # expert chosen, loads within binomial spread of T*k/E, activations ~N(0,1)
    import oracle
    T = 2048
    x, wr, b = synth.make_router_inputs("prefill8k", T=T)
    xf = synth.bf16_bits_to_f32(x)
    assert abs(float(xf.mean())) < 0.01 and abs(float(xf.std()) - 1.0) < 0.02
    idx, _ = oracle.select(oracle.router_logits(x, wr), b, 6)
    counts = np.bincount(idx.ravel(), minlength=256)
    mean = T * 6 / 256
    assert counts.min() > 0
    assert counts.max() < mean + 6 * np.sqrt(mean) and counts.min() > mean - 6 * np.sqrt(mean)
    # the same activations drawn i.i.d. leave the low-bias experts unchosen
    idx_iid, _ = oracle.select(oracle.router_logits(synth.make_x(T, 4096), wr), b, 6)
    assert (np.bincount(idx_iid.ravel(), minlength=256) == 0).sum() > 20


def test_zipf_router_gives_skewed_load():
    import oracle
    x, wr, b = synth.make_router_inputs("decode64")
    idx, _ = oracle.select(oracle.router_logits(x, wr), b, 6)
    counts = np.bincount(idx.ravel(), minlength=256)
    distinct = int((counts > 0).sum())
    assert 90 <= distinct <= 150
    assert counts.max() >= 25
