"""Float64 CPU oracle for the DeepSeek Sparse Attention (DSA) hot path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the C-ABI library and its Python binding) never calls it, and it shares no
code, constants or tables with the HIP kernels.

What it computes, stage by stage, in the order the pages give:

1. Lightning indexer.  "DeepSeek-V3.2: Pushing the Frontier of Open Large
   Language Models" (r.nikiv.dev summary), section "How DSA Works": the indexer
   scores a query against every key, cheaply, in FP8.  The ivugangingo.com
   article on DeepSeek-V3.2, section "Sparse attention with almost linear
   long-context costs": a few low-precision indexer heads run on every token
   pair.  The pages give no formula; this oracle uses
       score(t, s) = sum_j w[t, j] * ReLU(q[t, j, :] . k[s, :])
   over the causal pairs s <= pos(t), with q and k the e4m3fn bytes times
   their per-token fp32 scales, evaluated in float64.
2. Fine-grained selector.  Same two sections: keep the top-k key positions per
   query (k = 2048 on the pages).  Ties at the k-th value go to the lowest
   position; the result is listed in ascending position and padded with -1
   when fewer than k candidates exist.
3. Sparse attention.  Same sections, and "Deepseek V3.2 Frontier"
   (skillmd.com), section "Implementation" for the stage order (score, top-k,
   gather, softmax-weighted sum): MQA/MLA over the selected rows only.  All
   heads of a token share one latent KV row per key; the key is the whole
   row (latent + rope), the value its latent part.
3b. Prefill mode.  The threadnavigator.com thread (first tweet): separate
   attention modes for prefill and decode.  Read as MLA's per-head form:
   each head has its own key (decompressed part + shared rotary part) and
   value, over the same selected set.
4. Indexer alignment loss (training).  ivugangingo.com article, section
   "DeepSeek sparse attention pre-training continues": the indexer is trained
   with a KL loss towards the attention's distribution, over all causal keys
   in the dense warm-up and over the selected keys afterwards.  The loss of a
   token is KL(head-summed, L1-normalised attention probabilities || softmax
   of the indexer scores), with its gradient taken with respect to the scores,
   and that gradient carried back through the indexer to q, w and k.

Readings where the pages are silent or garbled:
the indexer formula and FP8 format; causality (a key is visible iff its
position <= the query's); the skillmd pseudo-code applies softmax to the
indexer scores, whereas the ivugangingo article runs a separate MQA/MLA path
on the selected set -- the oracle follows the article; the value is the
latent part of the row; -0.0 and +0.0 compare equal.

Nothing here is tuned; every step is the plain definition.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# FP8 e4m3fn decoding (OCP 8-bit floating point, E4M3 "fn" variant)
# ---------------------------------------------------------------------------
def e4m3fn_decode(codes) -> np.ndarray:
    """Decode OCP e4m3fn bytes to float64 by the format's closed form.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
    field 0 encodes subnormals (-1)^s * 2^-6 * m/8; otherwise the value is
    (-1)^s * 2^(e-7) * (1 + m/8).  S.1111.111 is NaN; there is no infinity,
    so the largest finite magnitude is 2^8 * 1.75 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)


def dequantize(codes, scales) -> np.ndarray:
    """Per-token dequantisation: decoded bytes times one fp32 scale per leading row."""
    x = e4m3fn_decode(codes)
    s = np.asarray(scales, dtype=np.float64).reshape((-1,) + (1,) * (x.ndim - 1))
    return x * s


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64: the bits are the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Stage 1: lightning indexer
# ---------------------------------------------------------------------------
def indexer_row(q_row: np.ndarray, w_row: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Scores of one query against the keys it can see.

    q_row [H_I, d_I] and keys [n, d_I] are dequantised float64; w_row [H_I].
    Returns sum_j w[j] * max(0, q[j] . k[s]) for each of the n keys.
    """
    dots = q_row @ keys.T                       # [H_I, n]: per-head dot products
    return w_row @ np.maximum(dots, 0.0)        # ReLU, then the w-weighted head sum


def indexer_scores(q, w, k, pos) -> list[np.ndarray]:
    """Causal indexer scores for a set of query rows.

    q [R, H_I, d_I], w [R, H_I], k [S, d_I] float64 (already dequantised);
    pos[r] is the query's position in its sequence.  Row r sees keys
    0..pos[r]; the result is a list of R float64 arrays of length pos[r]+1.
    """
    return [indexer_row(q[r], w[r], k[: int(pos[r]) + 1]) for r in range(len(pos))]


# ---------------------------------------------------------------------------
# Stage 2: fine-grained top-k selector
# ---------------------------------------------------------------------------
def topk_select(scores_row, k: int) -> np.ndarray:
    """Positions of the k largest scores of one causal row, ascending, -1 padded.

    Candidates are positions 0..n-1 (n = len(scores_row)).  The order is
    score descending, then position ascending (ties at the threshold go to the
    lowest position); the first m = min(k, n) are kept and listed in
    ascending position.  -0.0 and +0.0 are equal under this order.
    """
    s = np.asarray(scores_row, dtype=np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))      # primary key: -score, secondary: position
    m = min(k, n)
    out = np.full(k, -1, dtype=np.int64)
    out[:m] = np.sort(order[:m])
    return out


# ---------------------------------------------------------------------------
# Stage 3: sparse MQA/MLA attention over the selected rows
# ---------------------------------------------------------------------------
def sparse_attention_row(q_row, kv, idx, scale: float, d_latent: int):
    """Attention of one token's H heads over its selected latent KV rows.

    q_row [H, D] and kv [S, D] float64 (D = latent + rope); idx [k] positions
    into kv, -1 entries skipped.  logits[h, i] = scale * q[h] . kv[idx_i];
    p = softmax over i; out[h] = sum_i p[h, i] * kv[idx_i, :d_latent];
    lse[h] = log sum_i exp(logits[h, i]) (natural log).
    Returns (out [H, d_latent], lse [H]).  With no valid index the output is 0
    and the lse is -inf.
    """
    idx = np.asarray(idx)
    sel = idx[idx >= 0]
    H = q_row.shape[0]
    if sel.size == 0:
        return np.zeros((H, d_latent)), np.full(H, -np.inf)
    rows = kv[sel]                              # [m, D] gathered rows
    logits = scale * (q_row @ rows.T)           # [H, m]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    den = e.sum(axis=1, keepdims=True)
    out = (e @ rows[:, :d_latent]) / den
    lse = mx[:, 0] + np.log(den[:, 0])
    return out, lse


# ---------------------------------------------------------------------------
# Stage 3, prefill mode: per-head keys and values
# ---------------------------------------------------------------------------
# The threadnavigator.com thread on DeepSeek-V3.2 (first tweet) notes that the
# model runs different attention modes for disaggregated prefill and decode.
# The pages give no shapes.  The reading used here is MLA's two forms of the
# same attention: the form of stage 3 (queries taken into the latent space,
# one shared latent + rope row per key) serves decode; for prefill every head
# has its own key -- a part decompressed from the latent, followed by the
# rotary key that all heads share -- and its own value, and the query of a
# head is as wide as its key.  The selector's set restricts the keys as a
# mask: each valid position of a row counts once.
def mha_attention_row(q_row, k_nope, k_rope, v, idx, scale: float, kv_len: int):
    """Prefill-mode attention of one token's H heads over its selected keys.

    q_row [H, dn + dr]; k_nope [S, H, dn]; k_rope [S, dr]; v [S, H, dv]
    (float64, rows = key positions of the token's sequence); idx [k]
    positions.  sel = the distinct entries of idx in [0, kv_len), ascending.
    logits[h, i] = scale * (q_row[h, :dn] . k_nope[sel_i, h] + q_row[h, dn:] . k_rope[sel_i]);
    out[h] = sum_i softmax_i(logits[h]) * v[sel_i, h]; lse[h] = log sum_i exp(logits[h, i]).
    Returns (out [H, dv], lse [H]); with nothing selected, 0 and -inf.
    """
    idx = np.asarray(idx)
    sel = np.unique(idx[(idx >= 0) & (idx < kv_len)])
    H, dn = q_row.shape[0], k_nope.shape[2]
    if sel.size == 0:
        return np.zeros((H, v.shape[2])), np.full(H, -np.inf)
    out = np.zeros((H, v.shape[2]))
    lse = np.zeros(H)
    for h in range(H):
        keys = np.concatenate([k_nope[sel, h, :], k_rope[sel]], axis=1)   # [m, dn + dr]
        logits = scale * (keys @ q_row[h])
        mx = logits.max()
        e = np.exp(logits - mx)
        out[h] = (e @ v[sel, h, :]) / e.sum()
        lse[h] = mx + np.log(e.sum())
    return out, lse


def mha_attention_rows(q, k_nope, k_rope, v, idx, scale: float, kv_len: int):
    """mha_attention_row over the rows of one sequence: q [R, H, dn + dr],
    idx [R, k]; returns (out [R, H, dv], lse [R, H])."""
    outs, lses = zip(*(mha_attention_row(q[r], k_nope, k_rope, v, idx[r], scale, kv_len)
                       for r in range(len(q))))
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------
# Composition: indexer -> selector -> attention, per query row
# ---------------------------------------------------------------------------
def forward_rows(q, w, k, pos, q_attn, kv, topk: int, scale: float, d_latent: int):
    """DSA for a set of query rows of one sequence, in float64.

    q [R, H_I, d_I], w [R, H_I], k [S, d_I] dequantised; pos [R]; q_attn
    [R, H, D], kv [S, D].  Returns (scores list, idx [R, k], out [R, H,
    d_latent], lse [R, H]).
    """
    scores = indexer_scores(q, w, k, pos)
    idx = np.stack([topk_select(s, topk) for s in scores])
    outs, lses = zip(*(sparse_attention_row(q_attn[r], kv, idx[r], scale, d_latent)
                       for r in range(len(pos))))
    return scores, idx, np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------
# Stage 4 (training): indexer alignment loss
# ---------------------------------------------------------------------------
# ivugangingo.com article on DeepSeek-V3.2, section "DeepSeek sparse attention
# pre-training continues": during the dense warm-up only the indexer learns,
# through a Kullback-Leibler loss that pulls its distribution towards the
# dense attention's; in the sparse stage (k = 2048 selected keys per query)
# the indexer's gradients come only from that alignment loss, taken over the
# selected keys.  The pages give no formula; the readings used here:
#   * the attention "distribution" of a token is its per-head softmax
#     probabilities summed over the heads and L1-normalised over the keys;
#   * the indexer's distribution is the softmax of its scores over the same
#     keys (all causal keys in the warm-up, the selected set afterwards);
#   * the loss of a token is KL(attention || indexer), with the attention side
#     held fixed: its gradient is taken with respect to the indexer scores only.
def attention_target_row(q_row, kv, keys, scale: float) -> np.ndarray:
    """Head-summed, L1-normalised attention distribution of one token over `keys`.

    q_row [H, D] and kv [S, D] float64; keys [m] row indices into kv (m >= 1).
    For each head, p_h = softmax(scale * q_h . kv[keys]); the target is
    sum_h p_h divided by its total (which is H).
    """
    rows = kv[np.asarray(keys)]
    logits = scale * (q_row @ rows.T)                    # [H, m]
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    per_head = e / e.sum(axis=1, keepdims=True)          # each row sums to 1
    summed = per_head.sum(axis=0)
    return summed / summed.sum()


def indexer_kl_row(scores_sel, target):
    """KL(target || softmax(scores_sel)) and its gradient with respect to scores_sel.

    With q = softmax(scores_sel): loss = sum_i target_i * (log target_i - log q_i),
    terms with target_i = 0 being 0.  Since sum_i target_i = 1, the derivative
    of the loss with respect to scores_sel[i] is q_i - target_i.
    """
    s = np.asarray(scores_sel, dtype=np.float64)
    p = np.asarray(target, dtype=np.float64)
    mx = s.max()
    log_q = s - (mx + np.log(np.exp(s - mx).sum()))
    pos = p > 0
    loss = float(np.sum(p[pos] * (np.log(p[pos]) - log_q[pos])))
    return loss, np.exp(log_q) - p


def alignment_loss_rows(q_attn, kv, scores, pos, scale: float, idx=None):
    """Alignment loss of a set of query rows of one sequence, in float64.

    q_attn [R, H, D], kv [S, D]; scores: R score rows, row r holding at least
    pos[r] + 1 entries (the indexer's scores of that query, key position as
    index).  Dense warm-up form (idx None): row r's keys are 0..pos[r].
    Sparse form: idx [R, k] selected positions, -1 entries skipped (the others
    taken as given, as the attention takes them).
    Returns (loss [R], grads): grads[r] is the gradient over the row's keys --
    dense: an array of length pos[r] + 1; sparse: [k], aligned with idx[r],
    zero at the -1 entries.  A row with no key has loss 0.
    """
    losses, grads = [], []
    for r in range(len(pos)):
        row_scores = np.asarray(scores[r], dtype=np.float64)
        if idx is None:
            keys = np.arange(int(pos[r]) + 1)
        else:
            sel = np.asarray(idx[r])
            keys = sel[sel >= 0]
        if keys.size == 0:
            losses.append(0.0)
            grads.append(np.zeros(0 if idx is None else len(idx[r])))
            continue
        target = attention_target_row(q_attn[r], kv, keys, scale)
        loss, g = indexer_kl_row(row_scores[keys], target)
        losses.append(loss)
        if idx is None:
            grads.append(g)
        else:
            full = np.zeros(len(idx[r]))
            full[np.asarray(idx[r]) >= 0] = g
            grads.append(full)
    return np.array(losses), grads


# ---------------------------------------------------------------------------
# Stage 4b (training): backward of the lightning indexer
# ---------------------------------------------------------------------------
# The alignment loss's gradient on the scores flows into the indexer's inputs
# (same section of the ivugangingo.com article: only the indexer learns from
# that loss).  With the score of stage 1,
#     score(t, s) = sum_j w[t, j] * ReLU(z[t, j, s]),   z = q[t, j] . k[s]
# (q and k dequantised), and an upstream gradient g[t, s], the chain rule
# gives, taking the ReLU's derivative at 0 as 0:
#     dw[t, j] = sum_s g[t, s] * ReLU(z[t, j, s])
#     dq[t, j] = sum_s g[t, s] * w[t, j] * [z[t, j, s] > 0] * k[s]
#     dk[s]    = sum_t sum_j g[t, s] * w[t, j] * [z[t, j, s] > 0] * q[t, j]
def indexer_backward_row(q_row, w_row, keys, g):
    """Gradients of sum_i g[i] * score(keys[i]) for one query row.

    q_row [H_I, d_I], w_row [H_I], keys [m, d_I] (dequantised float64), g [m].
    Returns (dq [H_I, d_I], dw [H_I], dk [m, d_I]); dk[i] belongs to keys[i].
    """
    z = q_row @ keys.T                          # [H_I, m]
    dw = np.maximum(z, 0.0) @ g
    e = (z > 0) * w_row[:, None] * g[None, :]   # d score_i / d z[j, i], times g[i]
    return e @ keys, dw, e.T @ q_row


def indexer_backward_rows(q, w, k, pos, grads, idx=None):
    """Indexer backward for a set of query rows of one sequence, in float64.

    q [R, H_I, d_I], w [R, H_I], k [S, d_I] dequantised; pos [R].  grads are
    the upstream gradients on the scores: dense (idx None), row r is indexed
    by key position 0..pos[r]; sparse, row r is aligned with idx[r] (entries
    with idx -1 ignored).  Returns (dq [R, H_I, d_I], dw [R, H_I], dk [S, d_I]),
    dk summed over the rows.
    """
    R = len(pos)
    dq = np.zeros(q.shape)
    dw = np.zeros(w.shape)
    dk = np.zeros(k.shape)
    for r in range(R):
        g_row = np.asarray(grads[r], dtype=np.float64)
        if idx is None:
            keys = np.arange(int(pos[r]) + 1)
            g = g_row[: keys.size]
        else:
            sel = np.asarray(idx[r])
            ok = sel >= 0
            keys, g = sel[ok], g_row[: sel.size][ok]
        if keys.size == 0:
            continue
        dq[r], dw[r], dk_rows = indexer_backward_row(q[r], w[r], k[keys], g)
        np.add.at(dk, keys, dk_rows)
    return dq, dw, dk
