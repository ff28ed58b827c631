"""Pins for the oracle's sparse MQA/MLA attention.

With every causal position selected the method is dense causal attention, so
the oracle must agree with torch's scaled_dot_product_attention (float64,
is_causal) with the shared KV row expanded to all heads.  Closed-form special
cases (one selected row, zero query, a two-key hand example) and invariants
cover the rest.
"""
import math

import numpy as np
import torch

from oracle import sparse_attention_row, topk_select


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_full_selection_equals_dense_causal_sdpa():
    L, H, dl, dr = 37, 4, 12, 5
    D = dl + dr
    scale = 1.0 / math.sqrt(D)
    q, kv = _rand((L, H, D), 1), _rand((L, D), 2)
    k = 64                                           # k >= L: every causal key selected
    outs, lses = [], []
    for t in range(L):
        idx = topk_select(_rand(t + 1, 100 + t), k)  # arbitrary scores; all n kept
        o, l = sparse_attention_row(q[t], kv, idx, scale, dl)
        outs.append(o)
        lses.append(l)
    out, lse = np.stack(outs), np.stack(lses)
    Q = torch.from_numpy(q).permute(1, 0, 2)                         # [H, L, D]
    K = torch.from_numpy(kv)[None].expand(H, L, D)
    V = torch.from_numpy(kv[:, :dl])[None].expand(H, L, dl)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    logits = scale * (Q @ K.transpose(1, 2))
    mask = torch.triu(torch.ones(L, L, dtype=torch.bool), 1)
    ref_lse = torch.logsumexp(logits.masked_fill(mask, -math.inf), dim=-1).T
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_single_selected_row_returns_its_latent_part():
    H, dl, dr, S = 3, 8, 4, 10
    q, kv = _rand((H, dl + dr), 3), _rand((S, dl + dr), 4)
    idx = np.array([6, -1, -1])
    out, lse = sparse_attention_row(q, kv, idx, 0.3, dl)
    np.testing.assert_allclose(out, np.broadcast_to(kv[6, :dl], (H, dl)), atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * (q @ kv[6]), rtol=1e-14)


def test_zero_query_is_mean_of_selected_values():
    H, dl, dr, S = 2, 6, 2, 20
    kv = _rand((S, dl + dr), 5)
    idx = np.array([1, 4, 9, 17, -1, -1])
    out, lse = sparse_attention_row(np.zeros((H, dl + dr)), kv, idx, 1.0, dl)
    np.testing.assert_allclose(out[0], kv[[1, 4, 9, 17], :dl].mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(lse, np.log(4.0), rtol=1e-14)


def test_two_key_hand_example():
    # logits 0 and ln 3 -> weights 1/4 and 3/4; value = latent coordinate only
    kv = np.array([[0.0, 1.0, 0.0], [1.0, 0.0, 5.0]])   # d_latent = 2, d_rope = 1
    q = np.array([[0.0, 0.0, math.log(3.0) / 5.0]])
    out, lse = sparse_attention_row(q, kv, np.array([0, 1]), 1.0, 2)
    np.testing.assert_allclose(out[0], [0.75, 0.25], rtol=1e-14)
    np.testing.assert_allclose(lse[0], math.log(4.0), rtol=1e-14)


def test_index_order_and_padding_do_not_matter():
    H, dl, dr, S = 4, 10, 3, 30
    q, kv = _rand((H, dl + dr), 6), _rand((S, dl + dr), 7)
    a = sparse_attention_row(q, kv, np.array([2, 5, 11, 29, -1, -1]), 0.25, dl)
    b = sparse_attention_row(q, kv, np.array([29, -1, 11, 2, -1, 5]), 0.25, dl)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-14)


def test_rope_part_enters_logits_but_not_values():
    H, dl, dr, S = 2, 4, 3, 6
    q, kv = _rand((H, dl + dr), 8), _rand((S, dl + dr), 9)
    idx = np.arange(S)
    out1, lse1 = sparse_attention_row(q, kv, idx, 0.5, dl)
    kv2 = kv.copy()
    kv2[:, dl:] *= 2.0
    out2, lse2 = sparse_attention_row(q, kv2, idx, 0.5, dl)
    assert np.abs(lse1 - lse2).max() > 1e-6          # rope changes the logits ...
    q3 = q.copy()
    q3[:, dl:] = 0.0
    out3, _ = sparse_attention_row(q3, kv, idx, 0.5, dl)
    out4, _ = sparse_attention_row(q3, kv2, idx, 0.5, dl)
    np.testing.assert_allclose(out3, out4, atol=1e-14)  # ... but never the values
