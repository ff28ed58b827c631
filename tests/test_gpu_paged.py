"""Paged caches through the C ABI: every stage that reads the key or latent
KV caches gives the same result from block-table caches as from the packed
ones (bit-identical: the same arithmetic in the same order), and the oracle's
on the logical rows.  Block tables are shuffled, leave unused blocks, and in
one case place the used blocks past 4 GB of the latent cache.  The decode
workload at full size (64 sequences, 8K-128K contexts) also runs through the
paged forward and is checked against the oracle directly."""
import math

import numpy as np
import pytest
import torch

from sparse_attention_18_amd import binding as dsa
from sparse_attention_18_amd import workloads as wk
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

MED = wk.PREFILL_4K.scaled(seq_len=700, topk=256, heads=128)


def _announce(name):
    print(f"\n[paged] {name}", flush=True)


@pytest.mark.parametrize("bs", [64, 256])
def test_paged_indexer_decode_matches_packed(bs):
    wl = wk.DECODE_B64.scaled(decode_batch=6, ctx_min=100, ctx_max=3000)
    _announce(f"indexer decode B=6 block {bs}")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g = H.to_dev(inp)
    ref = H.run_indexer(prob, g)
    pg, kc, ksc, _ = H.make_paged(inp, bs, seed=bs)
    ld = prob.ld_scores()
    sc = torch.full_like(ref, float("nan"))
    dsa.indexer_scores_paged(prob, pg, g["q_fp8"], g["q_scale"], g["w"], kc, ksc, sc, ld)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(sc, nan=-7.0), torch.nan_to_num(ref, nan=-7.0))
    offs = inp["kv_offsets"]
    for b in range(wl.decode_batch):
        refs = H.oracle_scores_for_rows(inp, slice(b, b + 1), offs[b], [inp["q_pos0"][b]])
        H.check_indexer_rows(sc, refs, [b])


@pytest.mark.parametrize("bs,r0,r1", [(64, 448, 700), (128, 0, 700)])
def test_paged_indexer_prefill_matches_packed(bs, r0, r1):
    _announce(f"indexer prefill rows [{r0},{r1}) block {bs}")
    inp = wk.generate(MED)
    sub = {k: (v[r0:r1] if k in ("q_fp8", "q_scale", "w", "q") else
               v[:r1] if k in ("k_fp8", "k_scale", "kv") else v) for k, v in inp.items()}
    sub["kv_offsets"] = [0, r1]
    prob = dsa.Problem.from_workload(MED, inp, q_rows=slice(r0, r1), q_pos0=r0)
    g = H.to_dev(sub)
    ref = H.run_indexer(prob, g)
    pg, kc, ksc, _ = H.make_paged(sub, bs, seed=7)
    sc = torch.full_like(ref, float("nan"))
    dsa.indexer_scores_paged(prob, pg, g["q_fp8"], g["q_scale"], g["w"], kc, ksc, sc, prob.ld_scores())
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(sc, nan=-7.0), torch.nan_to_num(ref, nan=-7.0))
    # and the oracle on the logical rows: the first, the last and a spread between
    local = sorted({0, 1, (r1 - r0) // 3, (r1 - r0) // 2, r1 - r0 - 2, r1 - r0 - 1})
    for i in local:
        refs = H.oracle_scores_for_rows(sub, slice(i, i + 1), 0, [r0 + i])
        H.check_indexer_rows(sc, refs, [i])


def _attn_inputs(T, S, k, H_, dl, dr, seed, fill=None):
    g = torch.Generator().manual_seed(seed)
    D = dl + dr
    q = torch.randn(T, H_, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(S, D, generator=g).to(torch.bfloat16)
    idx = torch.full((T, k), -1, dtype=torch.int32)
    for t in range(T):
        m = fill(t) if fill else min(k, S)
        idx[t, :m] = torch.randperm(S, generator=g)[:m].sort().values.to(torch.int32)
    return q, kv, idx


@pytest.mark.parametrize("H_,dl,dr,pad_to,high", [(128, 512, 64, None, 0), (128, 512, 64, 264, 0),
                                                   (64, 512, 64, None, 0), (8, 64, 16, None, 0),
                                                   (128, 512, 64, None, 4_000_000)])
def test_paged_attention_matches_packed(H_, dl, dr, pad_to, high):
    """One sequence of S keys; T query tokens at its last positions."""
    _announce(f"attention H={H_} D={dl}+{dr} pad_to={pad_to} high_rows={high}")
    T, S, k = 24, 5000, 2048
    fills = [2048, 2048, 1, 5, 31, 32, 33, 100, 1000, 2047, 0, 64] * 2
    q, kv, idx = _attn_inputs(T, S, k, H_, dl, dr, seed=H_ + dl, fill=lambda t: fills[t])
    if pad_to:
        q = torch.cat([q, torch.zeros(pad_to - T, H_, dl + dr, dtype=q.dtype)])
        idx = torch.cat([idx, torch.full((pad_to - T, k), -1, dtype=idx.dtype)])
    Tp = q.shape[0]
    scale = 1 / math.sqrt(dl + dr)
    prob = dsa.Problem(q_offsets=[0, Tp], kv_offsets=[0, S], q_pos0=[S - Tp], idx_heads=4,
                       idx_dim=32, heads=H_, d_latent=dl, d_rope=dr, topk=k, softmax_scale=scale)
    nws = dsa.workspace_bytes(prob, dsa.WS_ATTN)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    qd, kvd, idd = q.cuda(), kv.cuda(), idx.cuda()
    out_ref = torch.empty(Tp, H_, dl, dtype=torch.bfloat16, device="cuda")
    lse_ref = torch.empty(Tp, H_, dtype=torch.float32, device="cuda")
    dsa.sparse_attn(prob, qd, kvd, idd, out_ref, lse_ref, workspace=ws)
    fake = {"kv_offsets": [0, S], "kv": kv, "k_fp8": torch.zeros(S, 32, dtype=torch.uint8),
            "k_scale": torch.ones(S)}
    pg, _, _, kvc = H.make_paged(fake, 64, seed=3, high_base_rows=high)
    out = torch.full_like(out_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    dsa.sparse_attn_paged(prob, pg, qd, kvc, idd, out, lse, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    assert torch.equal(lse, lse_ref)
    rows = [t for t in range(T) if fills[t] > 0]
    H.check_attention_rows(out[:T], lse[:T], q, kv, idx, rows[:6], [0] * 6, scale, dl)


def test_paged_forward_decode_matches_packed():
    wl = wk.DECODE_B64.scaled(decode_batch=8, ctx_min=3000, ctx_max=40000)
    _announce("forward decode B=8 ctx 3000..40000 block 64")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g = H.to_dev(inp)
    B = wl.decode_batch
    ws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_FORWARD), dtype=torch.uint8, device="cuda")
    outs = []
    for paged in (False, True):
        out = torch.empty(B, wl.heads, wl.d_latent, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, wl.heads, dtype=torch.float32, device="cuda")
        idx = torch.empty(B, wl.topk, dtype=torch.int32, device="cuda")
        if paged:
            pg, kc, ksc, kvc = H.make_paged(inp, 64, seed=11)
            dsa.forward_paged(prob, pg, g["q_fp8"], g["q_scale"], g["w"], kc, ksc, g["q"], kvc, out,
                              lse, idx, ws)
        else:
            dsa.forward(prob, g["q_fp8"], g["q_scale"], g["w"], g["k_fp8"], g["k_scale"], g["q"],
                        g["kv"], out, lse, idx, ws)
        torch.cuda.synchronize()
        outs.append((out, lse, idx))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_paged_forward_decode_full_size_against_the_oracle():
    """The decode workload at full size (64 sequences, contexts 8K-128K)
    through dsa_forward_paged over shuffled 64-row blocks, checked against the
    oracle directly: indexer scores of 8 sequences, every row's selection
    (bit-exact against the oracle selector on the GPU's own scores) and every
    row's attention."""
    wl = wk.DECODE_B64
    _announce("forward decode B=64 ctx 8K..128K, paged (block 64), against the oracle")
    inp = wk.generate(wl, device="cuda")
    prob = dsa.Problem.from_workload(wl, inp, device="cuda")
    B = wl.decode_batch
    ws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_FORWARD), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, wl.heads, wl.d_latent, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, wl.heads, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, wl.topk, dtype=torch.int32, device="cuda")
    pg, kc, ksc, kvc = H.make_paged(inp, 64, seed=21)
    dsa.forward_paged(prob, pg, inp["q_fp8"], inp["q_scale"], inp["w"], kc, ksc, inp["q"], kvc, out, lse,
                      idx, ws)
    torch.cuda.synchronize()
    del kc, ksc, kvc
    ld = prob.ld_scores()
    scores = ws[: B * ld * 4].view(torch.float32).view(B, ld)      # dsa_forward keeps them first
    offs = [int(x) for x in inp["kv_offsets"]]
    pos = [int(x) for x in inp["q_pos0"]]
    for b in (0, 1, 17, 31, 40, 50, 62, 63):
        refs = H.oracle_scores_for_rows(inp, slice(b, b + 1), offs[b], [pos[b]])
        H.check_indexer_rows(scores, refs, [b])
    rows = list(range(B))
    H.check_topk_rows(idx, scores, rows, [p + 1 for p in pos], wl.topk)
    H.check_attention_rows(out, lse, inp["q"], inp["kv"], idx, rows, offs[:-1], wl.softmax_scale, wl.d_latent)
