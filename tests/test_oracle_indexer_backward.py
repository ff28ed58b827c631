"""Pins for the oracle's indexer backward (training stage).

The gradients must be the derivatives of sum_s g[t, s] * score(t, s) with the
score computed by the oracle's own stage-1 function (pinned on its own):
central finite differences check every input.  The score is piecewise
linear in each input, so away from a ReLU kink the differences are exact up
to rounding.  Further: the chain through the alignment loss, linearity in g,
zero weights, accumulation of a key's gradient over rows, the sparse form
over every position against the dense form, and a one-head closed form.
"""
import numpy as np
import pytest

from oracle import (alignment_loss_rows, indexer_backward_row, indexer_backward_rows,
                    indexer_row)


def _case(seed, R=3, H=4, d=6, S=9):
    g = np.random.default_rng(seed)
    return (g.standard_normal((R, H, d)), g.random((R, H)), g.standard_normal((S, d)),
            np.array([2, 5, 8])[:R], [g.standard_normal(S) for _ in range(R)])


def _objective(q, w, k, pos, grads):
    return sum(float(indexer_row(q[r], w[r], k[: pos[r] + 1]) @ grads[r][: pos[r] + 1])
               for r in range(len(pos)))


@pytest.mark.parametrize("seed", [1, 2])
def test_gradients_are_finite_differences_of_the_scores(seed):
    q, w, k, pos, grads = _case(seed)
    dq, dw, dk = indexer_backward_rows(q, w, k, pos, grads)
    h = 1e-6
    for arr, grad in ((q, dq), (w, dw), (k, dk)):
        flat = arr.reshape(-1)
        gflat = grad.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            fp = _objective(q, w, k, pos, grads)
            flat[i] = old - h
            fm = _objective(q, w, k, pos, grads)
            flat[i] = old
            assert gflat[i] == pytest.approx((fp - fm) / (2 * h), abs=1e-6), (arr.shape, i)


def test_chain_through_the_alignment_loss():
    """d(loss)/dw by finite differences of loss(indexer(q, w, k)) equals the
    backward fed with the loss's gradient on the scores."""
    rng = np.random.default_rng(3)
    H, d, S, Ha, D = 3, 5, 7, 2, 8
    q, w, k = rng.standard_normal((1, H, d)), rng.random((1, H)), rng.standard_normal((S, d))
    qa, kv = rng.standard_normal((1, Ha, D)), rng.standard_normal((S, D))
    pos = np.array([S - 1])

    def loss_of(wv):
        sc = indexer_row(q[0], wv[0], k)
        return alignment_loss_rows(qa, kv, [sc], pos, 0.5)[0][0]

    sc = indexer_row(q[0], w[0], k)
    _, g = alignment_loss_rows(qa, kv, [sc], pos, 0.5)
    _, dw, _ = indexer_backward_rows(q, w, k, pos, g)
    h = 1e-6
    for j in range(H):
        e = np.zeros_like(w)
        e[0, j] = h
        fd = (loss_of(w + e) - loss_of(w - e)) / (2 * h)
        assert dw[0, j] == pytest.approx(fd, abs=1e-7)


def test_linear_in_g_and_zero_weights():
    q, w, k, pos, grads = _case(4)
    a = indexer_backward_rows(q, w, k, pos, grads)
    b = indexer_backward_rows(q, w, k, pos, [2.5 * x for x in grads])
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, 2.5 * x, rtol=1e-13, atol=1e-15)
    dq, dw, dk = indexer_backward_rows(q, np.zeros_like(w), k, pos, grads)
    assert not dq.any() and not dk.any() and dw.any()


def test_key_gradient_accumulates_over_rows():
    q, w, k, pos, grads = _case(5)
    _, _, dk = indexer_backward_rows(q, w, k, pos, grads)
    total = np.zeros_like(k)
    for r in range(len(pos)):
        _, _, d1 = indexer_backward_rows(q[r:r + 1], w[r:r + 1], k, pos[r:r + 1], grads[r:r + 1])
        total += d1
    np.testing.assert_allclose(dk, total, rtol=1e-13, atol=1e-15)
    assert not dk[pos.max() + 1:].any()


def test_sparse_over_every_position_is_dense():
    q, w, k, pos, grads = _case(6)
    kk = 12
    idx = np.full((len(pos), kk), -1)
    g_sparse = []
    rng = np.random.default_rng(7)
    for r, p in enumerate(pos):
        slots = rng.permutation(kk)[: p + 1]
        idx[r, slots] = np.arange(p + 1)
        row = np.zeros(kk)
        row[slots] = grads[r][: p + 1]
        g_sparse.append(row)
    dense = indexer_backward_rows(q, w, k, pos, grads)
    sparse = indexer_backward_rows(q, w, k, pos, g_sparse, idx=idx)
    for x, y in zip(dense, sparse):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-15)


def test_one_head_closed_form():
    q = np.array([[1.0, -2.0, 0.5]])
    k = np.array([[2.0, 0.5, 4.0], [-1.0, 1.0, 0.0]])   # z = 3 (active), -3 (inactive)
    dq, dw, dk = indexer_backward_row(q, np.array([0.7]), k, np.array([2.0, 5.0]))
    np.testing.assert_allclose(dw, [2.0 * 3.0])
    np.testing.assert_allclose(dq, 2.0 * 0.7 * k[:1])
    np.testing.assert_allclose(dk, [2.0 * 0.7 * q[0], np.zeros(3)])


def test_relu_derivative_at_zero_is_zero():
    q = np.array([[1.0, 1.0]])
    k = np.array([[1.0, -1.0]])                           # z = 0 exactly
    dq, dw, dk = indexer_backward_row(q, np.array([1.0]), k, np.array([1.0]))
    assert not dq.any() and not dk.any() and not dw.any()
