"""Pins for the oracle's top-k selector.

The oracle sorts (score desc, position asc).  The pins use a different
formulation -- a position is selected iff fewer than m candidates beat it,
counting strictly larger scores plus equal scores at lower positions -- plus
torch.topk on tie-free rows, hand examples, and the structural invariants.
"""
import numpy as np
import pytest
import torch

from oracle import topk_select


def _brute(x, k):
    n = len(x)
    m = min(k, n)
    sel = []
    for s in range(n):
        rank = sum(1 for t in range(n) if x[t] > x[s] or (x[t] == x[s] and t < s))
        if rank < m:
            sel.append(s)
    return np.array(sel + [-1] * (k - len(sel)))


def _check_invariants(x, k, idx):
    n = len(x)
    m = min(k, n)
    valid = idx[idx >= 0]
    assert len(valid) == m
    assert (idx[:m] >= 0).all() and (idx[m:] == -1).all()      # -1 only at the tail
    assert (np.diff(valid) > 0).all()                          # strictly ascending
    assert valid.min() >= 0 and valid.max() < n
    unsel = np.setdiff1d(np.arange(n), valid)
    if len(unsel):
        thr = x[valid].min()
        assert x[unsel].max() <= thr
        eq_unsel = unsel[x[unsel] == thr]
        eq_sel = valid[x[valid] == thr]
        if len(eq_unsel):
            assert eq_unsel.min() > eq_sel.max()               # lowest positions win ties


def test_hand_examples():
    np.testing.assert_array_equal(topk_select([3, 1, 4, 1, 5, 9, 2, 6], 3), [4, 5, 7])
    np.testing.assert_array_equal(topk_select([2, 5, 5, 1, 5], 2), [1, 2])
    np.testing.assert_array_equal(topk_select([2, 5, 5, 1, 5], 3), [1, 2, 4])
    np.testing.assert_array_equal(topk_select([7.0], 4), [0, -1, -1, -1])
    np.testing.assert_array_equal(topk_select([1, 2, 3], 3), [0, 1, 2])


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny_rows(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    k = int(rng.integers(1, 24))
    # small integer values force many ties
    x = rng.integers(-3, 4, size=n).astype(np.float64)
    got = topk_select(x, k)
    np.testing.assert_array_equal(got, _brute(x, k))
    _check_invariants(x, k, got)


def test_matches_torch_topk_on_distinct_values():
    rng = np.random.default_rng(100)
    for n, k in [(50, 7), (300, 64), (1000, 999), (17, 17)]:
        x = rng.permutation(n).astype(np.float64) * 0.37 - 11.0
        ref = np.sort(torch.topk(torch.from_numpy(x), min(k, n)).indices.numpy())
        got = topk_select(x, k)
        np.testing.assert_array_equal(got[: len(ref)], ref)


def test_all_equal_row_takes_lowest_positions():
    np.testing.assert_array_equal(topk_select(np.full(10, 3.25), 4), [0, 1, 2, 3])


def test_signed_zero_ties_are_equal():
    x = np.array([-0.0, 0.0, -0.0, 0.0, -1.0, -0.0])
    np.testing.assert_array_equal(topk_select(x, 3), [0, 1, 2])
    x2 = np.array([-1.0, -0.0, 0.0, 0.0])
    np.testing.assert_array_equal(topk_select(x2, 2), [1, 2])


def test_invariants_on_continuous_rows():
    rng = np.random.default_rng(5)
    for n, k in [(100, 10), (4096, 2048), (5000, 2048), (64, 100)]:
        x = rng.standard_normal(n) * 32 + 144
        _check_invariants(x, k, topk_select(x, k))
