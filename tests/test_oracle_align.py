"""Pins for the oracle's indexer alignment loss (training stage).

The loss is KL(attention target || softmax(indexer scores)) per token, with
the target the head-summed, L1-normalised attention probabilities over the
token's keys.  Independent checks: the target reproduces the attention
oracle's head-averaged output (that oracle is pinned to torch's SDPA), a
one-head target is scipy's softmax, the KL value is scipy's relative entropy,
the gradient is the loss's finite-difference derivative, and closed forms for
a uniform target, a two-key hand example and a matched indexer.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import entropy

from oracle import (alignment_loss_rows, attention_target_row, indexer_kl_row,
                    sparse_attention_row)


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, H=6, D=20, S=40, d_latent=16):
    g = _rng(seed)
    return g.standard_normal((H, D)), g.standard_normal((S, D)), d_latent


def test_target_is_a_distribution():
    q, kv, _ = _case(1)
    t = attention_target_row(q, kv, np.arange(25), 0.3)
    assert t.shape == (25,)
    assert np.all(t >= 0)
    assert abs(t.sum() - 1.0) < 1e-12


@pytest.mark.parametrize("seed", [2, 3])
def test_target_reproduces_head_averaged_attention_output(seed):
    # mean_h out_h = sum_s target_s V_s; with fewer keys than latent dims and
    # random rows, V has full row rank, so this fixes the target uniquely.
    q, kv, dl = _case(seed, H=5, D=24, S=30, d_latent=20)
    keys = np.array([3, 7, 11, 12, 19, 25, 29])
    out, _ = sparse_attention_row(q, kv, keys, 0.25, dl)
    t = attention_target_row(q, kv, keys, 0.25)
    np.testing.assert_allclose(out.mean(axis=0), t @ kv[keys, :dl], rtol=0, atol=1e-12)
    sol, *_ = np.linalg.lstsq(kv[keys, :dl].T, out.mean(axis=0), rcond=None)
    np.testing.assert_allclose(sol, t, rtol=0, atol=1e-10)


def test_one_head_target_is_softmax():
    q, kv, _ = _case(4, H=1)
    keys = np.arange(0, 40, 3)
    ref = softmax(0.5 * (kv[keys] @ q[0]))
    np.testing.assert_allclose(attention_target_row(q, kv, keys, 0.5), ref, rtol=1e-12, atol=0)


def test_kl_is_scipy_relative_entropy():
    g = _rng(5)
    target = softmax(g.standard_normal(50) * 2)
    s = g.standard_normal(50) * 3
    loss, _ = indexer_kl_row(s, target)
    assert loss == pytest.approx(entropy(target, softmax(s)), rel=1e-12)
    assert loss >= 0


def test_gradient_is_the_finite_difference_derivative():
    g = _rng(6)
    target = softmax(g.standard_normal(12))
    s = g.standard_normal(12) * 2
    _, grad = indexer_kl_row(s, target)
    h = 1e-6
    for i in range(12):
        e = np.zeros(12)
        e[i] = h
        fd = (indexer_kl_row(s + e, target)[0] - indexer_kl_row(s - e, target)[0]) / (2 * h)
        assert grad[i] == pytest.approx(fd, abs=1e-8)
    assert abs(grad.sum()) < 1e-12      # both distributions sum to 1


def test_matched_indexer_has_zero_loss_and_gradient():
    g = _rng(7)
    target = softmax(g.standard_normal(30))
    loss, grad = indexer_kl_row(np.log(target) + 17.5, target)
    assert abs(loss) < 1e-12
    assert np.abs(grad).max() < 1e-12


def test_zero_query_gives_uniform_target_closed_form():
    _, kv, _ = _case(8)
    q = np.zeros((4, 20))
    keys = np.arange(10)
    t = attention_target_row(q, kv, keys, 0.3)
    np.testing.assert_allclose(t, np.full(10, 0.1), rtol=0, atol=1e-15)
    s = _rng(9).standard_normal(10)
    loss, grad = indexer_kl_row(s, t)
    logq = np.log(softmax(s))
    assert loss == pytest.approx(-math.log(10) - logq.mean(), rel=1e-12)
    np.testing.assert_allclose(grad, softmax(s) - 0.1, atol=1e-15)


def test_two_key_hand_example():
    # one head, equal logits -> target (1/2, 1/2); scores (0, ln 3) -> indexer (1/4, 3/4)
    q = np.zeros((1, 4))
    kv = np.ones((2, 4))
    t = attention_target_row(q, kv, np.array([0, 1]), 1.0)
    loss, grad = indexer_kl_row(np.array([0.0, math.log(3.0)]), t)
    assert loss == pytest.approx(0.5 * math.log(4.0 / 3.0), rel=1e-14)
    np.testing.assert_allclose(grad, [-0.25, 0.25], atol=1e-15)


def test_scores_shift_invariance():
    g = _rng(10)
    target = softmax(g.standard_normal(20))
    s = g.standard_normal(20) * 5
    a = indexer_kl_row(s, target)
    b = indexer_kl_row(s + 123.0, target)
    assert a[0] == pytest.approx(b[0], rel=1e-10)
    np.testing.assert_allclose(a[1], b[1], atol=1e-12)


def test_sparse_with_every_key_selected_is_dense():
    q, kv, _ = _case(11, H=3, S=20)
    qa = np.stack([q, q * 0.5, -q])
    pos = np.array([4, 11, 19])
    scores = [_rng(12 + r).standard_normal(20) * 2 for r in range(3)]
    k = 24
    idx = np.full((3, k), -1)
    for r, p in enumerate(pos):
        idx[r, : p + 1] = np.arange(p + 1)
    ld, gd = alignment_loss_rows(qa, kv, scores, pos, 0.2)
    ls, gs = alignment_loss_rows(qa, kv, scores, pos, 0.2, idx=idx)
    np.testing.assert_allclose(ld, ls, rtol=1e-13)
    for r, p in enumerate(pos):
        np.testing.assert_allclose(gs[r][: p + 1], gd[r], atol=1e-15)
        assert np.all(gs[r][p + 1:] == 0)


def test_sparse_skips_minus_one_anywhere_and_keeps_slots():
    q, kv, _ = _case(13, H=2, S=12)
    scores = [_rng(14).standard_normal(12)]
    idx = np.array([[5, -1, 0, 9, -1, 3]])
    loss, grads = alignment_loss_rows(q[None], kv, scores, np.array([11]), 0.4, idx=idx)
    keys = np.array([5, 0, 9, 3])
    ref_loss, ref_g = indexer_kl_row(scores[0][keys], attention_target_row(q, kv, keys, 0.4))
    assert loss[0] == pytest.approx(ref_loss, rel=1e-14)
    np.testing.assert_allclose(grads[0], [ref_g[0], 0, ref_g[1], ref_g[2], 0, ref_g[3]], atol=1e-16)


def test_row_without_keys_has_zero_loss():
    q, kv, _ = _case(15, H=2, S=8)
    loss, grads = alignment_loss_rows(q[None], kv, [np.zeros(8)], np.array([7]), 0.4,
                                      idx=np.full((1, 4), -1))
    assert loss[0] == 0.0 and np.all(grads[0] == 0) and grads[0].shape == (4,)
