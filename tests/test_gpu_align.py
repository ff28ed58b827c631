"""GPU parity of the indexer alignment loss (dsa_indexer_align_loss) against
the float64 oracle.

The loss takes the indexer scores, the selected indices and the attention's
lse; here those come from the library's own stages on seeded inputs (the
oracle is then run on the same scores and indices, as for the selector), or
are built in the test.  Both forms are covered: the sparse form over the
selected keys and the dense warm-up form over every causal key, on the MFMA
path (H = 32, 64, 128 with 576-wide rows) and the small-shape path, with
ragged last tiles, packed multi-sequence batches, -1 entries anywhere and a
row with no key.  Tolerances are in tests/gpu_helpers.py."""
import numpy as np
import pytest
import torch

from sparse_attention_18_amd import binding as dsa
from sparse_attention_18_amd import workloads as wk
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"
MED = wk.PREFILL_4K.scaled(seq_len=700, topk=256, heads=128)


def _announce(name):
    print(f"[gpu-case] {name}", flush=True)


def _stages(wl, inp, prob, idx=None):
    """indexer -> top-k (unless idx is given) -> attention; returns device
    inputs, scores, idx and lse."""
    g = H.to_dev(inp)
    scores = H.run_indexer(prob, g)
    c = prob.c
    if idx is None:
        idx = torch.empty(c.total_q, c.topk, dtype=torch.int32, device=DEV)
        n = dsa.workspace_bytes(prob, dsa.WS_TOPK)
        dsa.topk(prob, scores, idx, workspace=torch.empty(n, dtype=torch.uint8, device=DEV) if n else None)
    out = torch.empty(c.total_q, c.heads, c.d_latent, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(c.total_q, c.heads, dtype=torch.float32, device=DEV)
    n = dsa.workspace_bytes(prob, dsa.WS_ATTN)
    dsa.sparse_attn(prob, g["q"], g["kv"], idx, out, lse,
                    workspace=torch.empty(n, dtype=torch.uint8, device=DEV) if n else None)
    torch.cuda.synchronize()
    return g, scores, idx, lse


def _loss(prob, g, lse, scores, idx, dense_ld=None):
    c = prob.c
    loss = torch.full((c.total_q,), float("nan"), dtype=torch.float32, device=DEV)
    width = c.topk if idx is not None else dense_ld
    grad = torch.full((c.total_q, width), float("nan"), dtype=torch.float32, device=DEV)
    dsa.indexer_align_loss(prob, g["q"], g["kv"], lse, scores, loss, grad, idx=idx)
    torch.cuda.synchronize()
    return loss, grad


def _rows(L, extra=24, seed=5):
    base = {0, 1, 2, 30, 31, 32, 33, L - 1}
    base.update(int(x) for x in np.random.default_rng(seed).integers(0, L, extra))
    return sorted(r for r in base if r < L)


@pytest.mark.parametrize("heads", [128, 64, 32])
def test_align_sparse_prefill(heads):
    wl = MED.scaled(heads=heads)
    _announce(f"align loss sparse prefill L={wl.seq_len} k={wl.topk} H={heads}")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g, scores, idx, lse = _stages(wl, inp, prob)
    loss, grad = _loss(prob, g, lse, scores, idx)
    rows = _rows(wl.seq_len) + [255, 256, 257, 400]
    rows = sorted(set(rows))
    H.check_align_rows(loss, grad, inp["q"], inp["kv"], scores, rows, [0] * len(rows),
                       [wl.seq_len] * len(rows), rows, wl.softmax_scale, idx=idx)
    assert torch.isfinite(loss).all() and bool((loss >= -1e-4).all())


def test_align_sparse_broad_indexer_distribution():
    """The synthetic indexer puts nearly all of its mass on a few keys; with the
    scores scaled down its softmax spreads over the set, so the gradient's both
    terms matter.  The loss takes any scores array."""
    wl = MED
    _announce("align loss sparse, scores x 0.02")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g, scores, idx, lse = _stages(wl, inp, prob)
    small = scores * 0.02
    loss, grad = _loss(prob, g, lse, small, idx)
    rows = _rows(wl.seq_len, seed=9)
    H.check_align_rows(loss, grad, inp["q"], inp["kv"], small, rows, [0] * len(rows),
                       [wl.seq_len] * len(rows), rows, wl.softmax_scale, idx=idx)
    # gradients of a row sum to zero (both distributions sum to one)
    gs = grad[torch.as_tensor(rows, device=DEV)].double().sum(dim=1).abs().max().item()
    assert gs < 1e-5


def test_align_dense_warmup():
    """Dense form: every causal key.  lse comes from the sparse attention with
    k >= L, which is dense causal attention; entries past pos stay untouched."""
    wl = MED.scaled(seq_len=300, topk=512)
    _announce("align loss dense warm-up L=300")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g, scores, idx, lse = _stages(wl, inp, prob)
    ld = 320
    loss_d, grad_d = _loss(prob, g, lse, scores, None, dense_ld=ld)
    rows = list(range(0, 300, 7)) + [298, 299]
    H.check_align_rows(loss_d, grad_d, inp["q"], inp["kv"], scores, rows, [0] * len(rows),
                       [300] * len(rows), rows, wl.softmax_scale, idx=None)
    gd = grad_d.cpu()
    for r in range(300):
        assert torch.isnan(gd[r, r + 1:]).all() and torch.isfinite(gd[r, : r + 1]).all()
    # the sparse form over all positions is the same loss
    loss_s, grad_s = _loss(prob, g, lse, scores, idx)
    np.testing.assert_allclose(loss_s.cpu().numpy(), loss_d.cpu().numpy(), rtol=1e-4, atol=1e-5)
    gs = grad_s.cpu()
    for r in (0, 1, 100, 299):
        np.testing.assert_allclose(gs[r, : r + 1].numpy(), gd[r, : r + 1].numpy(), rtol=0,
                                   atol=1e-6 + 1e-4 * gd[r, : r + 1].abs().max().item())


def test_align_custom_indices_with_gaps_and_an_empty_row():
    wl = MED.scaled(seq_len=500, topk=96)
    _announce("align loss sparse, -1 anywhere, empty row")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    L, k = wl.seq_len, wl.topk
    rng = np.random.default_rng(3)
    idx_np = np.full((L, k), -1, dtype=np.int32)
    for r in range(L):
        m = min(r + 1, int(rng.integers(1, k + 1)))
        sel = rng.choice(r + 1, size=m, replace=False)
        slots = rng.choice(k, size=m, replace=False)
        idx_np[r, slots] = sel
    idx_np[17] = -1                      # a row without any key
    idx = torch.as_tensor(idx_np, device=DEV)
    g, scores, idx, lse = _stages(wl, inp, prob, idx=idx)
    loss, grad = _loss(prob, g, lse, scores, idx)
    rows = _rows(L, seed=4) + [17]
    rows = sorted(set(rows))
    H.check_align_rows(loss, grad, inp["q"], inp["kv"], scores, rows, [0] * len(rows),
                       [L] * len(rows), rows, wl.softmax_scale, idx=idx)
    assert loss[17].item() == 0.0 and bool((grad[17] == 0).all())
    gaps = torch.as_tensor(idx_np < 0, device=DEV)
    assert bool((grad[gaps] == 0).all())


def test_align_packed_batch_of_sequences():
    """Several sequences of one query each (the decode layout), ragged lengths."""
    wl = wk.DECODE_B64.scaled(decode_batch=6, ctx_min=40, ctx_max=1500, topk=256)
    _announce("align loss packed batch B=6")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g, scores, idx, lse = _stages(wl, inp, prob)
    loss, grad = _loss(prob, g, lse, scores, idx)
    offs, pos = inp["kv_offsets"], inp["q_pos0"]
    rows = list(range(6))
    lens = [offs[b + 1] - offs[b] for b in rows]
    H.check_align_rows(loss, grad, inp["q"], inp["kv"], scores, rows, offs[:-1], lens, pos,
                       wl.softmax_scale, idx=idx)
    ld = prob.ld_scores()
    loss_d, grad_d = _loss(prob, g, _dense_lse(prob, g), scores, None, dense_ld=ld)
    H.check_align_rows(loss_d, grad_d, inp["q"], inp["kv"], scores, rows, offs[:-1], lens, pos,
                       wl.softmax_scale, idx=None)


def _dense_lse(prob, g):
    """lse of dense causal attention for a one-query-per-sequence batch: the
    sparse attention over every position 0..pos (k = max_kv_len here)."""
    c = prob.c
    B = c.batch
    pos = prob.q_pos0_list
    k = max(p + 1 for p in pos)
    dprob = dsa.Problem(q_offsets=prob.q_offsets_list, kv_offsets=prob.kv_offsets_list,
                        q_pos0=pos, idx_heads=c.idx_heads, idx_dim=c.idx_dim, heads=c.heads,
                        d_latent=c.d_latent, d_rope=c.d_rope, topk=k, softmax_scale=c.softmax_scale)
    idx = torch.full((B, k), -1, dtype=torch.int32)
    for b, p in enumerate(pos):
        idx[b, : p + 1] = torch.arange(p + 1, dtype=torch.int32)
    out = torch.empty(B, c.heads, c.d_latent, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, c.heads, dtype=torch.float32, device=DEV)
    n = dsa.workspace_bytes(dprob, dsa.WS_ATTN)
    dsa.sparse_attn(dprob, g["q"], g["kv"], idx.to(DEV), out, lse,
                    workspace=torch.empty(n, dtype=torch.uint8, device=DEV) if n else None)
    torch.cuda.synchronize()
    return lse


@pytest.mark.parametrize("wl", [wk.TINY_PREFILL, MED.scaled(seq_len=200, heads=16, topk=64)],
                         ids=["tiny_H8_D80", "H16_D576"])
def test_align_small_shape_path(wl):
    _announce(f"align loss small path {wl.name} H={wl.heads} D={wl.d_qk}")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g, scores, idx, lse = _stages(wl, inp, prob)
    L = wl.seq_len
    rows = list(range(L)) if L <= 256 else _rows(L)
    loss, grad = _loss(prob, g, lse, scores, idx)
    H.check_align_rows(loss, grad, inp["q"], inp["kv"], scores, rows, [0] * len(rows), [L] * len(rows),
                       rows, wl.softmax_scale, idx=idx)
    if wl.topk >= L:
        # k >= L: the attention lse is dense, so the warm-up form applies too
        loss_d, grad_d = _loss(prob, g, lse, scores, None, dense_ld=prob.ld_scores())
        H.check_align_rows(loss_d, grad_d, inp["q"], inp["kv"], scores, rows, [0] * len(rows),
                           [L] * len(rows), rows, wl.softmax_scale, idx=None)


def test_align_last_chunk_of_128k_prefill():
    """The launch the training-stage bench times: the last 4096-row chunk of
    the 128K prefill (2048 selected keys per row), sampled rows."""
    wl = wk.CHUNKED_PREFILL_128K
    _announce("align loss 128K prefill, last chunk")
    inp = wk.generate(wl, device=DEV)
    L, C = wl.seq_len, wl.chunk
    r0 = L - C
    sl = slice(r0, L)
    prob = dsa.Problem.from_workload(wl, inp, device=DEV, q_rows=sl, q_pos0=r0)
    sub = dict(inp)
    for key in ("q_fp8", "q_scale", "w", "q"):
        sub[key] = inp[key][sl]
    g, scores, idx, lse = _stages(wl, sub, prob)
    loss, grad = _loss(prob, g, lse, scores, idx)
    rows = [0, 1, 31, 32, 2047, 2048, 4095] + [int(x) for x in np.random.default_rng(7).integers(0, C, 5)]
    rows = sorted(set(rows))
    H.check_align_rows(loss, grad, sub["q"], inp["kv"], scores, rows, [0] * len(rows), [L] * len(rows),
                       [r0 + r for r in rows], wl.softmax_scale, idx=idx)
    assert torch.isfinite(loss).all() and torch.isfinite(grad).all()
