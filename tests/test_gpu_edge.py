"""Degenerate batches on the GPU, through every entry point, against the
oracle: a packed batch mixing sequences with no queries, no keys, a single
key and a few keys (fewer than k), at the MFMA shapes (128 heads x 576,
indexer 64 x 128); and problems with no query rows at all, which must return
without writing anything."""
import numpy as np
import pytest
import torch

from sparse_attention_18_amd import binding as dsa
from sparse_attention_18_amd import workloads as wk
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"
WL = wk.PREFILL_4K.scaled(topk=8)


def _announce(name):
    print(f"[gpu-case] {name}", flush=True)


def _inputs(q_lens, kv_lens, seed=1):
    """Seeded tensors for a packed batch; each sequence's queries sit at its
    last q_len positions."""
    g = torch.Generator().manual_seed(seed)
    Tq, Tk = sum(q_lens), sum(kv_lens)
    q8, qs = wk.quantize_rows_e4m3(torch.randn(max(Tq, 1), WL.idx_heads, WL.idx_dim, generator=g))
    k8, ks = wk.quantize_rows_e4m3(torch.randn(max(Tk, 1), WL.idx_dim, generator=g))
    inp = dict(q_fp8=q8[:Tq], q_scale=qs[:Tq], w=torch.rand(Tq, WL.idx_heads, generator=g),
               k_fp8=k8[:Tk], k_scale=ks[:Tk],
               q=torch.randn(Tq, WL.heads, WL.d_qk, generator=g).to(torch.bfloat16),
               kv=torch.randn(Tk, WL.d_qk, generator=g).to(torch.bfloat16))
    q_off, kv_off = [0], [0]
    for a, b in zip(q_lens, kv_lens):
        q_off.append(q_off[-1] + a)
        kv_off.append(kv_off[-1] + b)
    pos0 = [b - a for a, b in zip(q_lens, kv_lens)]
    inp.update(q_offsets=q_off, kv_offsets=kv_off, q_pos0=pos0)
    return inp


@pytest.mark.parametrize("two_pass", [False, True], ids=["atomic", "two_pass"])
def test_mixed_degenerate_batch_all_entry_points(two_pass):
    """Also the two-pass dk: 64-key blocks here straddle several sequences."""
    q_lens, kv_lens = [0, 3, 0, 1, 2, 5], [50, 3, 0, 1, 40, 6]
    _announce(f"degenerate batch q_lens {q_lens} kv_lens {kv_lens} two_pass={two_pass}")
    inp = _inputs(q_lens, kv_lens)
    prob = dsa.Problem.from_workload(WL, inp)
    g = H.to_dev(inp)
    c = prob.c
    scores = H.run_indexer(prob, g)
    idx = torch.full((c.total_q, c.topk), -7, dtype=torch.int32, device=DEV)
    n = dsa.workspace_bytes(prob, dsa.WS_TOPK)
    dsa.topk(prob, scores, idx, workspace=torch.empty(n, dtype=torch.uint8, device=DEV) if n else None)
    out = torch.empty(c.total_q, c.heads, c.d_latent, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(c.total_q, c.heads, dtype=torch.float32, device=DEV)
    n = dsa.workspace_bytes(prob, dsa.WS_ATTN)
    dsa.sparse_attn(prob, g["q"], g["kv"], idx, out, lse,
                    workspace=torch.empty(n, dtype=torch.uint8, device=DEV) if n else None)
    loss = torch.empty(c.total_q, dtype=torch.float32, device=DEV)
    grad = torch.empty(c.total_q, c.topk, dtype=torch.float32, device=DEV)
    dsa.indexer_align_loss(prob, g["q"], g["kv"], lse, scores, loss, grad, idx=idx)
    dq = torch.empty(c.total_q, c.idx_heads, c.idx_dim, dtype=torch.float32, device=DEV)
    dw = torch.empty(c.total_q, c.idx_heads, dtype=torch.float32, device=DEV)
    dk = torch.zeros(c.total_kv, c.idx_dim, dtype=torch.float32, device=DEV)
    ws = None
    if two_pass:
        ws = torch.full((dsa.workspace_bytes(prob, dsa.WS_INDEXER_BWD),), 0xFF, dtype=torch.uint8, device=DEV)
    dsa.indexer_backward(prob, g["q_fp8"], g["q_scale"], g["w"], g["k_fp8"], g["k_scale"], grad, dq, dw, dk,
                         idx=idx, workspace=ws)
    torch.cuda.synchronize()

    rows, positions, kv0s, lens = [], [], [], []
    for b in range(len(q_lens)):
        for i in range(q_lens[b]):
            rows.append(inp["q_offsets"][b] + i)
            positions.append(inp["q_pos0"][b] + i)
            kv0s.append(inp["kv_offsets"][b])
            lens.append(kv_lens[b])
    for i, r in enumerate(rows):
        ref = H.oracle_scores_for_rows(inp, slice(r, r + 1), kv0s[i], [positions[i]])
        H.check_indexer_rows(scores, ref, [r])
    H.check_topk_rows(idx, scores, rows, [p + 1 for p in positions], WL.topk)
    H.check_attention_rows(out, lse, inp["q"], inp["kv"], idx, rows, kv0s, WL.softmax_scale, WL.d_latent)
    H.check_align_rows(loss, grad, inp["q"], inp["kv"], scores, rows, kv0s, lens, positions, WL.softmax_scale,
                       idx=idx)
    gr = grad.cpu().double().numpy()
    ix = idx.cpu().numpy()
    dq_r, dq_b, dw_r, dw_b, dk_r, dk_b = H.indexer_backward_reference(inp, rows, positions, kv0s,
                                                                       [gr[r] for r in rows],
                                                                       [ix[r] for r in rows])
    H.check_within(dq[rows].cpu().numpy(), dq_r, dq_b, "dq")
    H.check_within(dw[rows].cpu().numpy(), dw_r, dw_b, "dw")
    keys = sorted(dk_r)
    dkg = dk.cpu().double().numpy()
    H.check_within(dkg[keys], np.stack([dk_r[x] for x in keys]), np.stack([dk_b[x] for x in keys]), "dk")
    # a one-key sequence: its only row selects position 0 and its loss is 0 (both
    # distributions are one point) up to the fp32 rounding of its score (|I| ~ 2^8,
    # so |I| * 2^-24 ~ 2e-5 in the exponent)
    r1 = inp["q_offsets"][3]
    assert ix[r1, 0] == 0 and (ix[r1, 1:] == -1).all()
    assert abs(loss[r1].item()) < 1e-4


def test_problems_without_query_rows_write_nothing():
    _announce("problems with no query rows")
    inp = _inputs([0, 0], [20, 0])
    prob = dsa.Problem.from_workload(WL, inp)
    g = H.to_dev(inp)
    dsa.indexer_scores(prob, g["q_fp8"], g["q_scale"], g["w"], g["k_fp8"], g["k_scale"],
                       torch.empty(0, 64, device=DEV), 64)
    dsa.topk(prob, torch.empty(0, 64, device=DEV), torch.empty(0, WL.topk, dtype=torch.int32, device=DEV), ld=64)
    dsa.sparse_attn(prob, g["q"], g["kv"], torch.empty(0, WL.topk, dtype=torch.int32, device=DEV),
                    torch.empty(0, WL.heads, WL.d_latent, dtype=torch.bfloat16, device=DEV))
    dk = torch.full((20, WL.idx_dim), 3.0, device=DEV)
    assert dsa.workspace_bytes(prob, dsa.WS_INDEXER_BWD) == 0
    for ws in (None, torch.empty(16, dtype=torch.uint8, device=DEV)):
        dsa.indexer_backward(prob, g["q_fp8"], g["q_scale"], g["w"], g["k_fp8"], g["k_scale"],
                             torch.empty(0, WL.topk, device=DEV),
                             torch.empty(0, WL.idx_heads, WL.idx_dim, device=DEV),
                             torch.empty(0, WL.idx_heads, device=DEV), dk,
                             idx=torch.empty(0, WL.topk, dtype=torch.int32, device=DEV), workspace=ws)
    torch.cuda.synchronize()
    assert bool((dk == 3.0).all())     # dk is only ever added to, and here by nothing
