"""Pins for the oracle's lightning indexer.

score(t, s) = sum_j w[t, j] * ReLU(q[t, j] . k[s]) over causal pairs.  Pinned
by a hand-worked closed-form example, by the special case H_I = 1, w = 1
against torch's matmul, and by invariants a wrong sign, dropped ReLU, swapped
operand or wrong head index would break.
"""
import numpy as np
import torch

from oracle import indexer_row, indexer_scores


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_worked_example():
    # Two heads with one-hot queries pick out one key coordinate each:
    # score = 2*max(k0, 0) + 3*max(k1, 0).
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.array([2.0, 3.0])
    keys = np.array([[1.0, 1.0], [-1.0, 2.0], [3.0, -4.0], [-1.0, -1.0], [0.5, 0.25]])
    got = indexer_row(q, w, keys)
    np.testing.assert_array_equal(got, [5.0, 6.0, 6.0, 0.0, 1.75])


def test_single_head_unit_weight_is_relu_of_matmul():
    R, S, d = 6, 9, 5
    q, k = _rand((R, 1, d), 1), _rand((S, d), 2)
    w = np.ones((R, 1))
    pos = np.full(R, S - 1)
    got = np.stack(indexer_scores(q, w, k, pos))
    ref = torch.relu(torch.from_numpy(q[:, 0, :]) @ torch.from_numpy(k).T).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-14)


def test_causal_rows_have_pos_plus_one_entries_and_ignore_later_keys():
    R, S, H, d = 5, 12, 3, 4
    q, w, k = _rand((R, H, d), 3), np.abs(_rand((R, H), 4)), _rand((S, d), 5)
    pos = np.array([0, 3, 7, 8, 11])
    rows = indexer_scores(q, w, k, pos)
    assert [len(r) for r in rows] == [1, 4, 8, 9, 12]
    k2 = k.copy()
    k2[8:] = 1e6                                    # keys after position 7 changed
    rows2 = indexer_scores(q, w, k2, pos)
    for r in range(3):
        np.testing.assert_array_equal(rows[r], rows2[r])


def test_positive_homogeneity_in_query_and_key_scales():
    H, d, S = 4, 8, 10
    q, w, k = _rand((H, d), 6), np.abs(_rand((H,), 7)), _rand((S, d), 8)
    base = indexer_row(q, w, k)
    np.testing.assert_allclose(indexer_row(2.5 * q, w, k), 2.5 * base, rtol=1e-13)
    alpha = np.linspace(0.5, 3.0, S)
    np.testing.assert_allclose(indexer_row(q, w, k * alpha[:, None]), base * alpha, rtol=1e-13)


def test_relu_drops_negative_dots():
    H, d, S = 3, 6, 7
    q = np.abs(_rand((H, d), 9))
    k = np.abs(_rand((S, d), 10))                   # every dot product positive
    w = np.ones(H)
    assert (indexer_row(q, w, k) > 0).all()
    np.testing.assert_array_equal(indexer_row(q, w, -k), np.zeros(S))


def test_linear_in_w_and_head_permutation_invariant():
    H, d, S = 5, 7, 11
    q, k = _rand((H, d), 11), _rand((S, d), 12)
    w1, w2 = _rand((H,), 13), _rand((H,), 14)
    np.testing.assert_allclose(indexer_row(q, w1 + w2, k),
                               indexer_row(q, w1, k) + indexer_row(q, w2, k), atol=1e-12)
    perm = np.array([3, 0, 4, 1, 2])
    np.testing.assert_allclose(indexer_row(q[perm], w1[perm], k), indexer_row(q, w1, k),
                               atol=1e-12)


def test_one_hot_weight_selects_one_head():
    H, d, S = 4, 5, 6
    q, k = _rand((H, d), 15), _rand((S, d), 16)
    for j in range(H):
        w = np.zeros(H)
        w[j] = 1.0
        np.testing.assert_allclose(indexer_row(q, w, k), np.maximum(k @ q[j], 0.0), atol=1e-13)


def test_key_permutation_equivariance():
    H, d, S = 3, 4, 9
    q, w, k = _rand((H, d), 17), _rand((H,), 18), _rand((S, d), 19)
    perm = np.random.default_rng(20).permutation(S)
    np.testing.assert_allclose(indexer_row(q, w, k[perm]), indexer_row(q, w, k)[perm], atol=1e-13)
