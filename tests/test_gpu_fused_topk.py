"""GPU parity of the fused decode selection (dsa_forward_fused).

On problems the decode indexer serves (at most two query rows per sequence,
rows of at most 2^18 keys) dsa_forward_fused selects from what that indexer
leaves per 1024-key chunk (bin tables and bin-grouped keys) instead of from
scores.  Every row's indices must equal the oracle selector run on the GPU's
own scores bit for bit; those come from dsa_indexer_scores, whose decode
kernel computes them with the same arithmetic (the fused form only adds the
binning after it).  Indices, outputs and lse must also equal dsa_forward's
bit for bit.  Covered: rows of 1, 5, k - 1, k, k + 1 keys, a row one
chunk past k, long rows up to 2^18 keys; exact ties among the largest scores
(repeated key rows), rows whose scores are all equal (zero weights, or one
key row repeated: past 5632 keys the threshold's bin is then read from the
lists in global memory rather than LDS), negative scores, scores spread over
so many octaves that each chunk's bin table holds hundreds of entries, k = 1
and k = 4096, and the paged caches.  Attention on a few rows is checked against the oracle too, so the
selection feeds the rest of the path as before."""
import math

import numpy as np
import pytest
import torch

from sparse_attention_18_amd import binding as dsa
from sparse_attention_18_amd import workloads as wk
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"
WL = wk.DECODE_B64                # indexer 64 x 128 fp8, 128 heads x 576, k = 2048


def _announce(name):
    print(f"[gpu-case] {name}", flush=True)


def _inputs(lens, seed, mutate=None):
    """Decode inputs for sequences of the given cache lengths, one query each
    at the last position: indexer q/k N(0,1) quantised per token, w U(0,1),
    attention q/kv N(0,1) bf16 (the decode workload's laws).  `mutate(inp)`
    edits the host tensors before they go to the GPU."""
    gen = torch.Generator().manual_seed(seed)
    B, T = len(lens), int(sum(lens))
    q_fp8, q_scale = wk.quantize_rows_e4m3(torch.randn(B, WL.idx_heads, WL.idx_dim, generator=gen))
    k_f32 = torch.randn(T, WL.idx_dim, generator=gen)
    inp = dict(q_fp8=q_fp8, q_scale=q_scale, w=torch.rand(B, WL.idx_heads, generator=gen),
               k_f32=k_f32, q=torch.randn(B, WL.heads, WL.d_qk, generator=gen).to(torch.bfloat16),
               kv=torch.randn(T, WL.d_qk, generator=gen).to(torch.bfloat16),
               q_offsets=list(range(B + 1)), kv_offsets=[0] + list(np.cumsum(lens)),
               q_pos0=[n - 1 for n in lens])
    if mutate is not None:
        mutate(inp)
    inp["k_fp8"], inp["k_scale"] = wk.quantize_rows_e4m3(inp.pop("k_f32"))
    if "k_scale_factor" in inp:
        inp["k_scale"] = inp["k_scale"] * inp.pop("k_scale_factor")
    return inp


def _forward(inp, k=WL.topk, paged=None):
    prob = dsa.Problem(q_offsets=inp["q_offsets"], kv_offsets=inp["kv_offsets"], q_pos0=inp["q_pos0"],
                       idx_heads=WL.idx_heads, idx_dim=WL.idx_dim, heads=WL.heads, d_latent=WL.d_latent,
                       d_rope=WL.d_rope, topk=k, softmax_scale=WL.softmax_scale, device=DEV)
    g = H.to_dev(inp)
    B = prob.total_q
    out = torch.empty(B, WL.heads, WL.d_latent, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, WL.heads, dtype=torch.float32, device=DEV)
    idx = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    ws = torch.full((dsa.workspace_bytes(prob, dsa.WS_FORWARD_FUSED),), 0xFF, dtype=torch.uint8, device=DEV)
    pg = None
    if paged is None:
        kc, ksc, kvc = g["k_fp8"], g["k_scale"], g["kv"]
    else:
        pg, kc, ksc, kvc = H.make_paged(inp, paged, seed=3)
    dsa.forward_fused(prob, g["q_fp8"], g["q_scale"], g["w"], kc, ksc, g["q"], kvc, out, lse, idx, ws, pg=pg)
    # dsa_forward on the same inputs: bit-identical results
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    idx2 = torch.empty_like(idx)
    ws2 = torch.empty(dsa.workspace_bytes(prob, dsa.WS_FORWARD), dtype=torch.uint8, device=DEV)
    if pg is None:
        dsa.forward(prob, g["q_fp8"], g["q_scale"], g["w"], kc, ksc, g["q"], kvc, out2, lse2, idx2, ws2)
    else:
        dsa.forward_paged(prob, pg, g["q_fp8"], g["q_scale"], g["w"], kc, ksc, g["q"], kvc, out2, lse2,
                          idx2, ws2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "indices differ from dsa_forward's"
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "outputs differ from dsa_forward's"
    ld = prob.ld_scores()
    scores = torch.full((B, ld), float("nan"), dtype=torch.float32, device=DEV)
    if paged is None:
        dsa.indexer_scores(prob, g["q_fp8"], g["q_scale"], g["w"], g["k_fp8"], g["k_scale"], scores, ld)
    else:
        dsa.indexer_scores_paged(prob, pg, g["q_fp8"], g["q_scale"], g["w"], kc, ksc, scores, ld)
    torch.cuda.synchronize()
    return prob, scores, idx, out, lse


def _check(inp, k=WL.topk, attn_rows=(), paged=None):
    prob, scores, idx, out, lse = _forward(inp, k, paged)
    lens = [inp["kv_offsets"][b + 1] - inp["kv_offsets"][b] for b in range(prob.total_q)]
    H.check_topk_rows(idx, scores, list(range(prob.total_q)), lens, k)
    if attn_rows:
        rows = list(attn_rows)
        H.check_attention_rows(out, lse, inp["q"], inp["kv"].to(DEV), idx, rows,
                               [inp["kv_offsets"][r] for r in rows], WL.softmax_scale, WL.d_latent)
    return idx


LENS = [1, 5, 2047, 2048, 2049, 3072, 3073, 65537, 1 << 18]


def test_fused_selection_lengths_around_k_and_chunks():
    _announce(f"fused decode selection, lengths {LENS}")
    _check(_inputs(LENS, 1), attn_rows=(0, 4, 7, 8))


@pytest.mark.parametrize("k", [1, 4096])
def test_fused_selection_extreme_k(k):
    _announce(f"fused decode selection k={k}")
    _check(_inputs([1, 4095, 4096, 4097, 9000, 70000], 2), k=k)


def test_fused_selection_exact_ties():
    """A handful of key rows repeated at many positions: their scores are
    exactly equal, and several of them rank near the threshold."""
    def mutate(inp):
        off = inp["kv_offsets"]
        g = torch.Generator().manual_seed(9)
        for b in range(len(off) - 1):
            n = off[b + 1] - off[b]
            if n < 8:
                continue
            hot = inp["k_f32"][off[b]:off[b] + 4].clone() * 1.5
            at = torch.randperm(n, generator=g)[: n // 3] + off[b]
            inp["k_f32"][at] = hot[torch.arange(at.numel()) % 4]
    _announce("fused decode selection, repeated key rows")
    _check(_inputs([3000, 9000, 40000, 131072], 3, mutate), attn_rows=(1, 3))


def test_fused_selection_all_equal_and_negative_scores():
    """Sequence 0: one key row repeated (all scores equal: its 20000 keys all
    sit in the threshold's bin, more than LDS holds, so that bin is read from
    the lists in global memory); 1: zero weights (every score +0); 2:
    negative weights (negative scores); 3: a short all-equal row (5000 keys,
    in LDS)."""
    lens = [20000, 9000, 30000, 5000]

    def mutate(inp):
        off = inp["kv_offsets"]
        inp["k_f32"][off[0]:off[1]] = inp["k_f32"][off[0]]
        inp["w"][1] = 0.0
        inp["w"][2] = -inp["w"][2]
        inp["k_f32"][off[3]:off[4]] = inp["k_f32"][off[3] + 1]
    _announce("fused decode selection, all-equal, zero and negative scores")
    idx = _check(_inputs(lens, 4, mutate))
    # all-equal rows take their lowest positions
    for b in (0, 1, 3):
        assert torch.equal(idx[b].cpu(), torch.arange(WL.topk, dtype=torch.int32))


def test_fused_selection_wide_score_range():
    """Key scales spread over 2^-40 .. 2^40: a chunk's scores then fall in
    hundreds of bins of an eighth of an octave (long bin tables)."""
    lens = [6000, 50000]

    def mutate(inp):
        g = torch.Generator().manual_seed(5)
        T = inp["k_f32"].shape[0]
        inp["k_scale_factor"] = torch.exp2(torch.rand(T, generator=g) * 80.0 - 40.0)
    _announce("fused decode selection, scores over 80 octaves")
    _check(_inputs(lens, 5, mutate))


def test_fused_selection_paged_matches_packed():
    _announce("fused decode selection over paged caches (128-row blocks)")
    inp = _inputs([2049, 7000, 33000, 100000], 6)
    idx_packed = _check(inp)
    idx_paged = _check(inp, paged=128)
    assert torch.equal(idx_packed, idx_paged)


def test_fused_refuses_what_it_does_not_serve():
    """Rows longer than 2^18 keys (the selection's LDS bitmap) and prefill
    problems are refused before anything is enqueued."""
    inp = _inputs([5000, (1 << 18) + 1], 7)
    prob = dsa.Problem(q_offsets=inp["q_offsets"], kv_offsets=inp["kv_offsets"], q_pos0=inp["q_pos0"],
                       idx_heads=WL.idx_heads, idx_dim=WL.idx_dim, heads=WL.heads, d_latent=WL.d_latent,
                       d_rope=WL.d_rope, topk=WL.topk, softmax_scale=WL.softmax_scale, device=DEV)
    with pytest.raises(dsa.DsaError) as e:
        dsa.workspace_bytes(prob, dsa.WS_FORWARD_FUSED)
    assert "262144" in str(e.value)
