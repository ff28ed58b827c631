"""GPU parity of the prefill-mode attention (dsa_sparse_attn_prefill).

The per-head form: each head has its own keys (128 decompressed + the 64-wide
rotary key shared by the heads) and values (128), over the selected set taken
as a mask.  Every compared row and head must match the float64 oracle
(mha_attention_row) on the GPU's own bf16 inputs within the attention bound
(max-abs 2e-2, relative Frobenius 1e-2; lse within 1e-3 of max(1, |lse|)).

Covered: a ragged single sequence (partial query block and key tile), packed
sequences given as chunks (q_pos0 > 0) with rows that select fewer than k
keys, repeated, negative and out-of-range entries and an empty row, rows that
select every causal key, head counts 1, 5, 8 and 128, and the 4096-token
prefill at full size on the selection the indexer and the top-k make."""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_18_amd import binding as dsa
from sparse_attention_18_amd import workloads as wk
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / math.sqrt(192.0)


def _announce(name):
    print(f"[gpu-case] {name}", flush=True)


def _selection(q_lens, kv_lens, q_pos0, k, seed, messy=False):
    """Per query row: up to k distinct causal positions, ascending, -1 padded.
    With `messy`, some rows also carry repeats, -5 and positions past the
    sequence, and the last row of the first sequence selects nothing."""
    rng = np.random.default_rng(seed)
    rows = []
    for b, (ql, kl, p0) in enumerate(zip(q_lens, kv_lens, q_pos0)):
        for i in range(ql):
            pos = p0 + i
            n = min(k, pos + 1) if rng.random() > 0.2 else int(rng.integers(1, min(k, pos + 1) + 1))
            sel = np.sort(rng.choice(pos + 1, size=n, replace=False))
            row = np.full(k, -1, dtype=np.int32)
            row[:n] = sel
            if messy and n + 3 <= k and i % 3 == 0:
                row[n:n + 3] = [sel[0], -5, kl + 7]
            if messy and b == 0 and i == ql - 1:
                row[:] = -1
            rows.append(row)
    return torch.from_numpy(np.stack(rows))


def _run(q_lens, kv_lens, q_pos0, heads, k, idx, seed):
    B = len(q_lens)
    q_off = [0] + list(np.cumsum(q_lens))
    kv_off = [0] + list(np.cumsum(kv_lens))
    inp = wk.mha_prefill_inputs(int(q_off[-1]), int(kv_off[-1]), heads, seed, device=DEV)
    prob = dsa.Problem(q_offsets=q_off, kv_offsets=kv_off, q_pos0=list(q_pos0), idx_heads=64, idx_dim=128,
                       heads=heads, d_latent=512, d_rope=64, topk=k, softmax_scale=SCALE, device=DEV)
    T = int(q_off[-1])
    out = torch.full((T, heads, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((T, heads), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.full((dsa.workspace_bytes(prob, dsa.WS_ATTN_PREFILL),), 0xA5, dtype=torch.uint8, device=DEV)
    idx_d = idx.to(DEV)
    dsa.sparse_attn_prefill(prob, inp["q"], inp["k_nope"], inp["k_rope"], inp["v"], idx_d, out, lse, ws)
    torch.cuda.synchronize()
    return inp, out, lse, q_off, kv_off


def _check(inp, out, lse, idx, rows, q_off, kv_off, q_pos0):
    """Oracle on the given packed rows (all heads)."""
    refs, lrefs = [], []
    for r in rows:
        b = int(np.searchsorted(q_off, r, side="right") - 1)
        k0, k1 = int(kv_off[b]), int(kv_off[b + 1])
        o, l = oracle.mha_attention_row(inp["q"][r].cpu().double().numpy(),
                                        inp["k_nope"][k0:k1].cpu().double().numpy(),
                                        inp["k_rope"][k0:k1].cpu().double().numpy(),
                                        inp["v"][k0:k1].cpu().double().numpy(),
                                        idx[r].numpy(), SCALE, k1 - k0)
        refs.append(o)
        lrefs.append(l)
    ref, lref = np.stack(refs), np.stack(lrefs)
    got = out[rows].cpu().double().numpy()
    lgot = lse[rows].cpu().double().numpy()
    max_abs = np.abs(got - ref).max()
    rel_f = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    beyond, row_ulps = H.bf16_rounding_split(got, ref)
    assert max_abs <= H.ATTN_MAX_ABS and rel_f <= H.ATTN_REL_F, \
        (f"prefill attention max-abs {max_abs:.3e} relF {rel_f:.3e} ({beyond:.3e} beyond the bf16 "
         f"output rounding; worst row {row_ulps:.2f} half-ulps)")
    fin = np.isfinite(lref)
    assert (np.isfinite(lgot) == fin).all(), "lse finiteness differs (rows with nothing selected)"
    if fin.any():
        assert np.abs(lgot[fin] - lref[fin]).max() <= 1e-3 * max(1.0, np.abs(lref[fin]).max())
    empty = ~fin.any(axis=1)
    assert np.all(got[empty] == 0)
    return max_abs, rel_f


@pytest.mark.parametrize("heads", [1, 5])
def test_prefill_mha_single_ragged_sequence(heads):
    """300 rows and keys: a partial second query block and a partial key tile."""
    _announce(f"prefill-mode attention, L=300, heads={heads}, k=64")
    q_lens, kv_lens, p0 = [300], [300], [0]
    idx = _selection(q_lens, kv_lens, p0, 64, seed=1)
    inp, out, lse, qo, ko = _run(q_lens, kv_lens, p0, heads, 64, idx, seed=2)
    _check(inp, out, lse, idx, list(range(300)), qo, ko, p0)


def test_prefill_mha_packed_chunks_with_messy_rows():
    """Three sequences given as chunks of their last rows (q_pos0 > 0): 260
    rows at 740..999 of a 1000-key sequence, 70 rows of a 70-key one, 1 row at
    512 of a 513-key one; repeats, -5, positions past the sequence and an
    empty row in the mix."""
    q_lens, kv_lens, p0 = [260, 70, 1], [1000, 70, 513], [740, 0, 512]
    _announce("prefill-mode attention, packed chunks, heads=8, k=128")
    idx = _selection(q_lens, kv_lens, p0, 128, seed=3, messy=True)
    inp, out, lse, qo, ko = _run(q_lens, kv_lens, p0, 8, 128, idx, seed=4)
    _check(inp, out, lse, idx, list(range(int(qo[-1]))), qo, ko, p0)


def test_prefill_mha_every_causal_key_selected():
    """k >= L: every row selects its whole causal prefix (dense causal MHA)."""
    _announce("prefill-mode attention, dense causal, L=200, heads=8")
    L = 200
    idx = torch.full((L, 256), -1, dtype=torch.int32)
    for t in range(L):
        idx[t, :t + 1] = torch.arange(t + 1, dtype=torch.int32)
    inp, out, lse, qo, ko = _run([L], [L], [0], 8, 256, idx, seed=5)
    _check(inp, out, lse, idx, list(range(L)), qo, ko, [0])


def test_prefill_mha_4k_full_size():
    """The 4096-token prefill at 128 heads, on the selection dsa_forward's
    indexer and top-k make for that workload (k = 2048); sampled rows across
    the query blocks, every head."""
    wl = wk.PREFILL_4K
    _announce(f"prefill-mode attention at full size, {wl.name}")
    gen_inp = wk.generate(wl, device=DEV)
    prob = dsa.Problem.from_workload(wl, gen_inp, device=DEV)
    L = wl.seq_len
    ld = prob.ld_scores()
    scores = torch.empty((L, ld), dtype=torch.float32, device=DEV)
    dsa.indexer_scores(prob, gen_inp["q_fp8"], gen_inp["q_scale"], gen_inp["w"], gen_inp["k_fp8"],
                       gen_inp["k_scale"], scores, ld)
    idx = torch.empty((L, wl.topk), dtype=torch.int32, device=DEV)
    tws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_TOPK), dtype=torch.uint8, device=DEV)
    dsa.topk(prob, scores, idx, ld, tws)
    del scores
    torch.cuda.synchronize()
    idx_cpu = idx.cpu()
    inp = wk.mha_prefill_inputs(L, L, wl.heads, seed=wl.seed + 100, device=DEV)
    out = torch.full((L, wl.heads, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((L, wl.heads), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_ATTN_PREFILL), dtype=torch.uint8, device=DEV)
    dsa.sparse_attn_prefill(prob, inp["q"], inp["k_nope"], inp["k_rope"], inp["v"], idx, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rows = [0, 1, 255, 256, 1023, 2046, 2047, 2048, 2049, 3071, 3584, 4095]
    _check(inp, out, lse, idx_cpu, rows, [0, L], [0, L], [0])


def test_prefill_mha_null_lse_and_no_rows():
    """lse is optional (same out bit for bit without it); a problem with no
    query rows returns without launching anything."""
    _announce("prefill-mode attention, lse NULL and an empty problem")
    q_lens, kv_lens, p0 = [150], [150], [0]
    idx = _selection(q_lens, kv_lens, p0, 32, seed=8)
    inp, out, lse, qo, ko = _run(q_lens, kv_lens, p0, 4, 32, idx, seed=9)
    prob = dsa.Problem(q_offsets=qo, kv_offsets=ko, q_pos0=p0, idx_heads=64, idx_dim=128, heads=4,
                       d_latent=512, d_rope=64, topk=32, softmax_scale=SCALE, device=DEV)
    out2 = torch.full_like(out, float("nan"))
    ws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_ATTN_PREFILL), dtype=torch.uint8, device=DEV)
    dsa.sparse_attn_prefill(prob, inp["q"], inp["k_nope"], inp["k_rope"], inp["v"], idx.to(DEV), out2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    empty = dsa.Problem(q_offsets=[0, 0], kv_offsets=[0, 150], q_pos0=[0], idx_heads=64, idx_dim=128, heads=4,
                        d_latent=512, d_rope=64, topk=32, softmax_scale=SCALE, device=DEV)
    z = torch.empty(0, 4, 192, dtype=torch.bfloat16, device=DEV)
    zo = torch.empty(0, 4, 128, dtype=torch.bfloat16, device=DEV)
    zi = torch.empty(0, 32, dtype=torch.int32, device=DEV)
    ws0 = torch.empty(dsa.workspace_bytes(empty, dsa.WS_ATTN_PREFILL), dtype=torch.uint8, device=DEV)
    dsa.sparse_attn_prefill(empty, z, inp["k_nope"], inp["k_rope"], inp["v"], zi, zo, None, ws0)
    torch.cuda.synchronize()
