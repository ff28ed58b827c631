"""Pins for the oracle's prefill-mode (per-head) attention.

* MLA's two forms are one attention: with per-head keys decompressed from a
  latent by W_UK and values by W_UV, the per-head form must equal W_UV times
  the output of the shared-row form (the stage-3 oracle, itself pinned to
  torch's SDPA) on the query taken into the latent space by W_UK^T, with the
  same lse.  A wrong head index, a dropped rotary term, a swapped key/value
  or a misapplied scale all break this.
* With every causal key selected the form is dense causal multi-head
  attention: torch's scaled_dot_product_attention in float64.
* The selection is a set: padding, out-of-range entries and repeats change
  nothing; one selected key gives its value and its logit.
"""
import math

import numpy as np
import torch

from oracle import mha_attention_row, mha_attention_rows, sparse_attention_row


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_per_head_form_equals_absorbed_form_times_value_projection():
    S, H, dn, dr, dl, dv = 40, 3, 6, 4, 10, 5
    scale = 1.0 / math.sqrt(dn + dr)
    c, k_r = _rand((S, dl), 1), _rand((S, dr), 2)          # latent rows, rotary keys
    w_uk, w_uv = _rand((H, dn, dl), 3), _rand((H, dv, dl), 4)
    q = _rand((H, dn + dr), 5)
    k_nope = np.einsum("hnl,sl->shn", w_uk, c)              # [S, H, dn]
    v = np.einsum("hvl,sl->shv", w_uv, c)                   # [S, H, dv]
    q_abs = np.concatenate([np.einsum("hnl,hn->hl", w_uk, q[:, :dn]), q[:, dn:]], axis=1)
    kv = np.concatenate([c, k_r], axis=1)                   # [S, dl + dr]
    idx = np.array([3, 7, 8, 20, 21, 22, 39, -1, -1])
    out, lse = mha_attention_row(q, k_nope, k_r, v, idx, scale, S)
    out_lat, lse_abs = sparse_attention_row(q_abs, kv, idx, scale, dl)
    np.testing.assert_allclose(out, np.einsum("hvl,hl->hv", w_uv, out_lat), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_abs, rtol=1e-12, atol=1e-12)


def test_full_selection_equals_dense_causal_multihead_sdpa():
    L, H, dn, dr, dv = 29, 4, 8, 4, 6
    scale = 1.0 / math.sqrt(dn + dr)
    q, k_nope, k_r, v = _rand((L, H, dn + dr), 11), _rand((L, H, dn), 12), _rand((L, dr), 13), _rand((L, H, dv), 14)
    idx = np.full((L, 32), -1)
    for t in range(L):
        idx[t, : t + 1] = np.arange(t + 1)
    out, lse = mha_attention_rows(q, k_nope, k_r, v, idx, scale, L)
    Q = torch.from_numpy(q).permute(1, 0, 2)                                           # [H, L, dn+dr]
    K = torch.cat([torch.from_numpy(k_nope), torch.from_numpy(k_r)[:, None, :].expand(L, H, dr)], 2)
    K = K.permute(1, 0, 2).contiguous()
    V = torch.from_numpy(v).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    logits = scale * (Q @ K.transpose(1, 2))
    logits = logits.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).T.numpy(), rtol=1e-12, atol=1e-12)


def test_selection_is_a_set():
    S, H, dn, dr, dv = 16, 2, 4, 2, 3
    q, k_nope, k_r, v = _rand((H, dn + dr), 21), _rand((S, H, dn), 22), _rand((S, dr), 23), _rand((S, H, dv), 24)
    clean = mha_attention_row(q, k_nope, k_r, v, np.array([2, 5, 9]), 0.7, S)
    messy = mha_attention_row(q, k_nope, k_r, v, np.array([9, -1, 5, 2, 5, 16, 40, -3, 2]), 0.7, S)
    np.testing.assert_array_equal(clean[0], messy[0])
    np.testing.assert_array_equal(clean[1], messy[1])
    # kv_len cuts the set: position 9 is outside a 9-key sequence
    cut = mha_attention_row(q, k_nope, k_r, v, np.array([2, 5, 9]), 0.7, 9)
    ref = mha_attention_row(q, k_nope, k_r, v, np.array([2, 5]), 0.7, S)
    np.testing.assert_array_equal(cut[0], ref[0])


def test_one_key_and_no_key():
    S, H, dn, dr, dv = 8, 3, 4, 2, 5
    q, k_nope, k_r, v = _rand((H, dn + dr), 31), _rand((S, H, dn), 32), _rand((S, dr), 33), _rand((S, H, dv), 34)
    out, lse = mha_attention_row(q, k_nope, k_r, v, np.array([-1, 6, -1]), 0.5, S)
    np.testing.assert_allclose(out, v[6], rtol=1e-15)
    for h in range(H):
        z = 0.5 * (sum(q[h, i] * k_nope[6, h, i] for i in range(dn)) +
                   sum(q[h, dn + i] * k_r[6, i] for i in range(dr)))
        assert abs(lse[h] - z) < 1e-12
    out, lse = mha_attention_row(q, k_nope, k_r, v, np.array([-1, -1]), 0.5, S)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
