"""Tiling and repeat checks: a race on LDS or on the workspace shows up as
results that change with the work decomposition or from one run to the next.

* Each stage runs twice on the same inputs and must give the same bits (every
  kernel here reduces in a fixed order; none uses floating-point atomics).
* The same rows go through two decompositions the launcher picks by batch
  shape: a query chunk against the whole prefill (indexer query tiles and key
  splits), few rows against many (top-k row segments against one workgroup
  per row; attention key-range splits with a combine against one workgroup
  per token).  Selections must agree bit for bit; scores and outputs within
  the bounds the oracle comparisons use, since a different decomposition may
  round differently.  Both sides of every pair are also oracle-checked in
  the parity tests."""
import math

import numpy as np
import pytest
import torch

from sparse_attention_18_amd import binding as dsa
from sparse_attention_18_amd import workloads as wk
from tests import gpu_helpers as H
from tests import test_gpu_parity as P
from tests import test_gpu_prefill_mha as M

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[gpu-case] {name}", flush=True)


def _same_bits(a, b, what):
    a, b = a.cpu(), b.cpu()
    if a.dtype.is_floating_point:
        a, b = a.view(torch.int16 if a.element_size() == 2 else torch.int32), \
            b.view(torch.int16 if b.element_size() == 2 else torch.int32)
    diff = (a != b).sum().item()
    assert diff == 0, f"{what}: {diff} elements differ between two identical calls"


def test_indexer_repeat_and_chunk_tiling():
    wl = P.MED.scaled(seq_len=1500)
    L, r0 = wl.seq_len, 1024
    _announce(f"indexer L={L}: twice, and rows [{r0},{L}) as a chunk")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g = H.to_dev(inp)
    s1 = H.run_indexer(prob, g)
    s2 = H.run_indexer(prob, g)
    _same_bits(s1, s2, "prefill indexer scores")
    sub = {k: (v[r0:L] if k in ("q_fp8", "q_scale", "w", "q") else v) for k, v in inp.items()}
    pc = dsa.Problem.from_workload(wl, inp, q_rows=slice(r0, L), q_pos0=r0)
    sc = H.run_indexer(pc, H.to_dev(sub))
    a = s1[r0:L, :L].cpu().double()
    b = sc[:, :L].cpu().double()
    causal = ~torch.triu(torch.ones(L - r0, L, dtype=torch.bool), r0 + 1)
    peak = a[causal].abs().max().item()
    err = (a[causal] - b[causal]).abs().max().item()
    assert err <= 1e-3 * peak, f"chunk against whole prefill: {err:.3e} > 1e-3 x {peak:.3e}"


def test_topk_segmented_and_rowwise_agree_and_repeat():
    _announce("top-k: row segments against one workgroup per row, twice each")
    k = 2048
    rng = np.random.default_rng(21)
    lengths = [131072, 70001, 40000, 32768, 9000, 2049, 2048, 700]
    rows = [rng.standard_normal(n).astype(np.float32) * 32 + 144 for n in lengths]
    rows[2][1000:31000] = 7.0            # a long run of ties at one value
    n = len(lengths)
    _, seg1 = P._topk_on(rows, lengths, k)
    _, seg2 = P._topk_on(rows, lengths, k)
    _, row1 = P._topk_on(rows, lengths, k, pad_rows=600)
    _, row2 = P._topk_on(rows, lengths, k, pad_rows=600)
    _same_bits(seg1, seg2, "segmented top-k")
    _same_bits(row1[:n], row2[:n], "row-wise top-k")
    _same_bits(seg1, row1[:n], "segmented against row-wise top-k")


def test_attention_split_and_per_token_agree_and_repeat():
    _announce("attention: key-range splits against one workgroup per token, twice each")
    T, S, k = 16, 9000, 2048
    fills = [2048, 2048, 1, 33, 1000, 2047, 64, 2048] * 2
    q, kv, idx, scale = P._attn_case(128, 512, 64, T, S, k, seed=77, fill=lambda t: fills[t],
                                     scale=1 / math.sqrt(192))
    o_s1, l_s1 = P._run_attn(q, kv, idx, scale, 512, 64)
    o_s2, l_s2 = P._run_attn(q, kv, idx, scale, 512, 64)
    o_t1, l_t1 = P._run_attn(q, kv, idx, scale, 512, 64, pad_to=264)
    o_t2, l_t2 = P._run_attn(q, kv, idx, scale, 512, 64, pad_to=264)
    _same_bits(o_s1, o_s2, "split attention output")
    _same_bits(l_s1, l_s2, "split attention lse")
    _same_bits(o_t1, o_t2, "per-token attention output")
    _same_bits(l_t1, l_t2, "per-token attention lse")
    a, b = o_s1.float().cpu(), o_t1.float().cpu()
    max_abs = (a - b).abs().max().item()
    rel_f = ((a - b).norm() / b.norm().clamp_min(1e-30)).item()
    assert max_abs <= H.ATTN_MAX_ABS and rel_f <= H.ATTN_REL_F, (max_abs, rel_f)
    assert (l_s1.cpu() - l_t1.cpu()).abs().max().item() <= 1e-3 * max(1.0, l_t1.abs().max().item())


def test_prefill_mode_attention_repeat():
    _announce("prefill-mode attention twice on packed chunks")
    q_lens, kv_lens, q_pos0 = [300, 129], [300, 513], [0, 384]
    k = 256
    idx = M._selection(q_lens, kv_lens, q_pos0, k, seed=8, messy=True)
    _, o1, l1, _, _ = M._run(q_lens, kv_lens, q_pos0, 5, k, idx, seed=8)
    _, o2, l2, _, _ = M._run(q_lens, kv_lens, q_pos0, 5, k, idx, seed=8)
    _same_bits(o1, o2, "prefill-mode attention output")
    _same_bits(l1, l2, "prefill-mode attention lse")
