"""Pins of the oracle's expert selection and weights.

The pages give 256 routed experts with six active per token
("DeepSeek V4 Flash serving hardware", 01, "Sparse architecture") and an FP32
``ffn.gate.bias`` (model card, "Component precisions"; the FP32 -> BF16
downcast is recorded as a bug under "Upstream contributions").  Reading:
sigmoid score, bias added for selection only, ties to the lower index,
weights renormalised over the chosen experts.  Selection is checked by brute
force over every k-subset.
"""
import itertools

import numpy as np

import oracle


def _keys(logits, bias):
    s = oracle.sigmoid(logits)
    return (s + bias.astype(np.float32)).astype(np.float32), s


def _brute_topk(key_row, k):
    """The k-subset whose keys, sorted by (key desc, index asc), is
    lexicographically largest (larger key first, then smaller index)."""
    E = key_row.shape[0]
    best = None
    for sub in itertools.combinations(range(E), k):
        seq = sorted(sub, key=lambda e: (-float(key_row[e]), e))
        tag = [(float(key_row[e]), -e) for e in seq]
        if best is None or tag > best[0]:
            best = (tag, seq)
    return best[1]


def test_selection_matches_brute_force():
    rng = np.random.default_rng(11)
    cases = [(16, 2)] + [(E, k) for E in (5, 8, 12) for k in (1, 2, 3, 4)]
    for E, k in cases:
        T = 30
        logits = rng.standard_normal((T, E)).astype(np.float32) * 1.3
        bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
        idx, _ = oracle.select(logits, bias, k)
        key, _ = _keys(logits, bias)
        for t in range(T):
            assert list(idx[t]) == _brute_topk(key[t], k), (E, k, t)


def test_ties_go_to_the_lower_index():
    E, k = 12, 4
    logits = np.zeros((1, E), np.float32)
    bias = np.zeros(E, np.float32)
    logits[0, [3, 9, 5, 10]] = 2.0   # four equal keys
    idx, w = oracle.select(logits, bias, k)
    assert list(idx[0]) == [3, 5, 9, 10]
    assert np.all(w[0] == np.float32(0.25))


def test_fp32_bias_decides_where_bf16_would_not():
    # equal scores (0.5); biases 0.05 and 0.050001 differ by more than an fp32
    # ulp of the key (~6e-8 near 0.55) but round to the same bf16 (0.0500488...)
    E = 4
    logits = np.zeros((1, E), np.float32)
    b_lo = np.float32(0.05)
    b_hi = np.float32(0.050001)
    bias = np.array([b_lo, -1, -1, b_hi], np.float32)
    idx, _ = oracle.select(logits, bias, 1)
    assert idx[0, 0] == 3                      # fp32: expert 3 has the larger key
    bias_bf16 = bias.copy()
    bias_bf16[[0, 3]] = np.float32(0.0500488281)  # both round to the same bf16 value
    idx2, _ = oracle.select(logits, bias_bf16, 1)
    assert idx2[0, 0] == 0                     # the tie goes to the lower index


def test_weights_use_unbiased_scores_and_are_renormalised():
    rng = np.random.default_rng(4)
    E, k, T = 16, 4, 50
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    idx, w = oracle.select(logits, bias, k)
    s = oracle.sigmoid(logits).astype(np.float64)
    for t in range(T):
        sel = s[t, idx[t]]
        assert abs(w[t].astype(np.float64).sum() - 1.0) <= k * 2.0 ** -23
        assert np.allclose(w[t], sel / sel.sum(), rtol=3e-7, atol=0)
    # moving the bias without changing the chosen set leaves the weights alone
    bias2 = bias + np.float32(0.0)
    bias2[idx[0, 0]] += np.float32(0.01)
    idx2, w2 = oracle.select(logits[:1], bias2, k)
    if set(idx2[0]) == set(idx[0]):
        assert np.array_equal(np.sort(w2[0]), np.sort(w[0]))


def test_routed_scale_multiplies_the_weights():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((8, 16)).astype(np.float32)
    bias = np.zeros(16, np.float32)
    _, w1 = oracle.select(logits, bias, 3, 1.0)
    _, w2 = oracle.select(logits, bias, 3, 2.0)
    assert np.array_equal(w2, w1 * np.float32(2.0))


def test_slot_order_is_descending_key():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((40, 256)).astype(np.float32) * 1.3
    bias = rng.uniform(-0.1, 0.1, 256).astype(np.float32)
    idx, _ = oracle.select(logits, bias, 6)
    key, _ = _keys(logits, bias)
    for t in range(40):
        ks = key[t, idx[t]]
        assert np.all(np.diff(ks) <= 0)
        assert ks[-1] >= np.max(np.delete(key[t], idx[t]))
        assert len(set(idx[t])) == 6
