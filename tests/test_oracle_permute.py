"""Pins of the oracle's token permutation (stable counting sort by group).

The expert GEMM on the pages is "indexed": rows reach an expert through an
index list ("Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass
through the model", the Humming settings).  Reading: slots grouped by expert
with prefix-sum offsets, stable in flat slot order, the shared expert as the
last group.  Checked against numpy's stable argsort.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("T,E,k,ns", [(8, 16, 2, 1), (64, 256, 6, 1), (33, 16, 3, 0), (1, 256, 6, 1),
                                      (500, 8, 8, 1)])
def test_permute_matches_stable_argsort(T, E, k, ns):
    rng = np.random.default_rng(T * 31 + E)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    offsets, sorted_token, row_of_slot = oracle.permute(idx, E, ns)
    S = k + ns
    groups = np.concatenate([idx, np.full((T, ns), E, np.int32)], axis=1).reshape(-1)
    order = np.argsort(groups, kind="stable")
    assert np.array_equal(sorted_token, order // S)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(row_of_slot.reshape(-1), inv)
    counts = np.bincount(groups, minlength=E + ns)
    assert offsets[0] == 0 and offsets[-1] == T * S
    assert np.array_equal(np.diff(offsets), counts)
    # every row of group g points back at a slot routed to g
    for g in range(E + ns):
        for r in range(offsets[g], offsets[g + 1]):
            t = sorted_token[r]
            j = list(row_of_slot[t]).index(r)
            assert (idx[t, j] if j < k else E) == g


def test_shared_group_holds_every_token_in_order():
    T, E, k = 40, 16, 2
    rng = np.random.default_rng(2)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    offsets, sorted_token, row_of_slot = oracle.permute(idx, E, 1)
    assert np.array_equal(sorted_token[offsets[E]:offsets[E + 1]], np.arange(T))
    assert np.array_equal(row_of_slot[:, k], offsets[E] + np.arange(T))


def test_out_of_range_index_is_rejected():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 16]], np.int32), 16, 1)
