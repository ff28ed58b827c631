"""GPU parity of the indexer backward (dsa_indexer_backward) against the
float64 oracle.

The score gradient is either seeded synthetic values or the alignment loss's
own gradient; indices come from the library's top-k on seeded inputs, or are
built in the test.  dq and dw are compared row by row, dk (accumulated by
atomics over every row) key by key, within the bounds in tests/gpu_helpers.py.
Covered: the MFMA path (H_I = 64, d_I = 128) in both forms with ragged last
tiles, -1 entries anywhere (in any order) and an empty row; two chunk calls
adding into one dk; the fp32 path for other shapes; sampled rows of the last
chunk of the 128K prefill (with the gradient zero outside the sampled rows, so
that dk is known exactly); and a sequence longer than the two-pass
reduction's 4096-row scan window, the first chunk (key blocks split over
workgroups) and keys shared by every row.  Every sparse MFMA case runs with
dk by atomics and with the two-pass dk (a workspace given)."""
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


def _topk(prob, g):
    scores = H.run_indexer(prob, g)
    idx = torch.empty(prob.total_q, prob.c.topk, dtype=torch.int32, device=DEV)
    n = dsa.workspace_bytes(prob, dsa.WS_TOPK)
    dsa.topk(prob, scores, idx, workspace=torch.empty(n, dtype=torch.uint8, device=DEV) if n else None)
    torch.cuda.synchronize()
    return scores, idx


def _workspace(prob, two_pass):
    """The two-pass workspace, filled with NaN bytes: nothing may read what
    the call did not write."""
    if not two_pass:
        return None
    n = dsa.workspace_bytes(prob, dsa.WS_INDEXER_BWD)
    assert n > 0
    return torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)


def _backward(prob, g, grad, idx, dk=None, two_pass=False):
    c = prob.c
    dq = torch.full((c.total_q, c.idx_heads, c.idx_dim), float("nan"), dtype=torch.float32, device=DEV)
    dw = torch.full((c.total_q, c.idx_heads), float("nan"), dtype=torch.float32, device=DEV)
    if dk is None:
        dk = torch.zeros(c.total_kv, c.idx_dim, dtype=torch.float32, device=DEV)
    dsa.indexer_backward(prob, g["q_fp8"], g["q_scale"], g["w"], g["k_fp8"], g["k_scale"], grad, dq, dw,
                         dk, idx=idx, workspace=_workspace(prob, two_pass))
    torch.cuda.synchronize()
    return dq, dw, dk


def _check(inp, prob, rows, positions, kv0s, grad, idx, dq, dw, dk, all_rows=True):
    gr = grad.cpu().double().numpy()
    ix = idx.cpu().numpy() if idx is not None else None
    ref = H.indexer_backward_reference(inp, rows, positions, kv0s, [gr[r] for r in rows],
                                       None if ix is None else [ix[r] for r in rows])
    dq_r, dq_b, dw_r, dw_b, dk_r, dk_b = ref
    H.check_within(dq[rows].cpu().numpy(), dq_r, dq_b, "dq")
    H.check_within(dw[rows].cpu().numpy(), dw_r, dw_b, "dw")
    if all_rows:
        dkg = dk.cpu().double().numpy()
        keys = sorted(dk_r)
        H.check_within(dkg[keys], np.stack([dk_r[x] for x in keys]), np.stack([dk_b[x] for x in keys]), "dk")
        untouched = np.ones(dkg.shape[0], dtype=bool)
        untouched[keys] = False
        assert not dkg[untouched].any(), "dk rows no row selected must stay zero"


TWO_PASS = pytest.mark.parametrize("two_pass", [False, True], ids=["atomic", "two_pass"])


@TWO_PASS
@pytest.mark.parametrize("seed", [0, 1])
def test_backward_sparse_mfma(seed, two_pass):
    wl = MED
    _announce(f"indexer backward sparse L={wl.seq_len} k={wl.topk} seed={seed} two_pass={two_pass}")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g = H.to_dev(inp)
    _, idx = _topk(prob, g)
    gen = torch.Generator(device="cpu").manual_seed(100 + seed)
    grad = (torch.randn(prob.total_q, wl.topk, generator=gen) * 1e-3).to(DEV)
    grad[idx < 0] = float("nan")        # entries past the selection are never read
    dq, dw, dk = _backward(prob, g, grad, idx, two_pass=two_pass)
    L = wl.seq_len
    _check(inp, prob, list(range(L)), list(range(L)), [0] * L, torch.nan_to_num(grad), idx, dq, dw, dk)


def test_backward_dense_mfma():
    """The dense form ignores a workspace (its pairs are all causal keys)."""
    wl = MED.scaled(seq_len=300)
    _announce("indexer backward dense L=300")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g = H.to_dev(inp)
    ld = prob.ld_scores()
    gen = torch.Generator(device="cpu").manual_seed(7)
    grad = torch.randn(prob.total_q, ld, generator=gen) * 1e-3
    for r in range(300):
        grad[r, r + 1:] = float("nan")   # past pos: never read
    dq, dw, dk = _backward(prob, g, grad.to(DEV), None, two_pass=True)
    L = wl.seq_len
    _check(inp, prob, list(range(L)), list(range(L)), [0] * L, torch.nan_to_num(grad), None, dq, dw, dk)


@TWO_PASS
def test_backward_custom_indices_gaps_and_empty_row(two_pass):
    """Indices in random order (the two-pass form sorts them), a few keys
    listed twice in a row, k = 80 (not a multiple of the 64-key tile)."""
    wl = MED.scaled(seq_len=400, topk=80)
    _announce(f"indexer backward sparse, -1 anywhere, empty row, two_pass={two_pass}")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g = H.to_dev(inp)
    L, k = wl.seq_len, wl.topk
    rng = np.random.default_rng(11)
    idx_np = np.full((L, k), -1, dtype=np.int32)
    for r in range(L):
        m = min(r + 1, int(rng.integers(1, k + 1)))
        idx_np[r, rng.choice(k, size=m, replace=False)] = rng.choice(r + 1, size=m, replace=False)
    idx_np[5] = -1
    # a key listed twice in a row counts once per entry
    for r in (9, 150, 399):
        v = np.flatnonzero(idx_np[r] >= 0)
        assert len(v) >= 2
        idx_np[r, v[1]] = idx_np[r, v[0]]
    idx = torch.as_tensor(idx_np, device=DEV)
    grad = torch.as_tensor(rng.standard_normal((L, k)) * 1e-3, dtype=torch.float32, device=DEV)
    dq, dw, dk = _backward(prob, g, grad, idx, two_pass=two_pass)
    _check(inp, prob, list(range(L)), list(range(L)), [0] * L, grad, idx, dq, dw, dk)
    assert not dq[5].any() and not dw[5].any()


@pytest.mark.parametrize("form", ["atomic", "two_pass", "dense"])
def test_backward_zero_scales_and_zero_key(form):
    """Zero scales dequantise to zero vectors: z = 0 there, the ReLU's
    derivative is 0, and the gradients must be finite and match the oracle
    (a key whose scale is 0 but whose e4m3 bytes are not, a key whose bytes
    are all zero, and query rows whose scale is 0)."""
    wl = MED.scaled(seq_len=320)
    _announce(f"indexer backward, zero scales and a zero key row, {form}")
    inp = wk.generate(wl)
    for key in (0, 3, 40, 200, 319):
        inp["k_scale"][key] = 0.0
    inp["k_fp8"][77] = 0
    for row in (2, 150, 300):
        inp["q_scale"][row] = 0.0
    prob = dsa.Problem.from_workload(wl, inp)
    g = H.to_dev(inp)
    L = wl.seq_len
    gen = torch.Generator(device="cpu").manual_seed(5)
    if form == "dense":
        ld = prob.ld_scores()
        grad = (torch.randn(L, ld, generator=gen) * 1e-3).to(DEV)
        idx = None
    else:
        _, idx = _topk(prob, g)
        grad = (torch.randn(L, wl.topk, generator=gen) * 1e-3).to(DEV)
    dq, dw, dk = _backward(prob, g, grad, idx, two_pass=form == "two_pass")
    for name, t in (("dq", dq), ("dw", dw), ("dk", dk)):
        assert torch.isfinite(t).all(), f"{name} has non-finite entries"
    _check(inp, prob, list(range(L)), list(range(L)), [0] * L, grad, idx, dq, dw, dk)
    assert not dq[[2, 150, 300]].any(), "a zero query scale gives dq = 0"


@TWO_PASS
def test_backward_chunks_add_into_one_dk(two_pass):
    """Two chunk calls (rows [0, 300) and [300, 600)) adding into one dk give
    the single call's dk."""
    wl = MED.scaled(seq_len=600)
    _announce(f"indexer backward, two chunks into one dk, two_pass={two_pass}")
    inp = wk.generate(wl)
    g = H.to_dev(inp)
    prob = dsa.Problem.from_workload(wl, inp)
    _, idx = _topk(prob, g)
    gen = torch.Generator(device="cpu").manual_seed(3)
    grad = (torch.randn(600, wl.topk, generator=gen) * 1e-3).to(DEV)
    dq, dw, dk_all = _backward(prob, g, grad, idx, two_pass=two_pass)
    dk = torch.zeros_like(dk_all)
    for r0, r1 in ((0, 300), (300, 600)):
        sub = {key: (v[r0:r1] if key in ("q_fp8", "q_scale", "w", "q") else v) for key, v in g.items()}
        pc = dsa.Problem.from_workload(wl, inp, q_rows=slice(r0, r1), q_pos0=r0)
        sub["k_fp8"], sub["k_scale"] = g["k_fp8"][:r1], g["k_scale"][:r1]
        _backward(pc, sub, grad[r0:r1].contiguous(), idx[r0:r1].contiguous(), dk=dk[:r1], two_pass=two_pass)
    # both dk are checked against the oracle over every row
    _check(inp, prob, list(range(600)), list(range(600)), [0] * 600, grad, idx, dq, dw, dk)
    _check(inp, prob, list(range(600)), list(range(600)), [0] * 600, grad, idx, dq, dw, dk_all)


@pytest.mark.parametrize("wl", [wk.TINY_PREFILL, MED.scaled(seq_len=200, idx_heads=48, idx_dim=64, topk=64)],
                         ids=["tiny_HI4_d32", "HI48_d64"])
def test_backward_fp32_path(wl):
    _announce(f"indexer backward fp32 path H_I={wl.idx_heads} d_I={wl.idx_dim}")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g = H.to_dev(inp)
    _, idx = _topk(prob, g)
    L = wl.seq_len
    gen = torch.Generator(device="cpu").manual_seed(5)
    grad = (torch.randn(L, wl.topk, generator=gen) * 1e-3).to(DEV)
    dq, dw, dk = _backward(prob, g, grad, idx)
    _check(inp, prob, list(range(L)), list(range(L)), [0] * L, grad, idx, dq, dw, dk)
    ld = prob.ld_scores()
    gd = (torch.randn(L, ld, generator=gen) * 1e-3).to(DEV)
    dq, dw, dk = _backward(prob, g, gd, None)
    _check(inp, prob, list(range(L)), list(range(L)), [0] * L, gd, None, dq, dw, dk)


@TWO_PASS
def test_backward_of_the_alignment_loss_gradient(two_pass):
    """The composed training step: the alignment loss's gradient on the
    scores carried back through the indexer."""
    wl = MED.scaled(seq_len=500)
    _announce(f"indexer backward of the alignment loss gradient, two_pass={two_pass}")
    inp = wk.generate(wl)
    prob = dsa.Problem.from_workload(wl, inp)
    g = H.to_dev(inp)
    scores, idx = _topk(prob, g)
    c = prob.c
    out = torch.empty(c.total_q, c.heads, c.d_latent, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(c.total_q, c.heads, dtype=torch.float32, device=DEV)
    dsa.sparse_attn(prob, g["q"], g["kv"], idx, out, lse)
    loss = torch.empty(c.total_q, dtype=torch.float32, device=DEV)
    grad = torch.empty(c.total_q, c.topk, dtype=torch.float32, device=DEV)
    dsa.indexer_align_loss(prob, g["q"], g["kv"], lse, scores, loss, grad, idx=idx)
    dq, dw, dk = _backward(prob, g, grad, idx, two_pass=two_pass)
    L = wl.seq_len
    _check(inp, prob, list(range(L)), list(range(L)), [0] * L, grad, idx, dq, dw, dk)


@TWO_PASS
def test_backward_last_chunk_of_128k_prefill(two_pass):
    """The launch a training step makes per chunk, at full size: the last
    4096-row chunk against the 131072-key prefix.  The gradient is nonzero on
    a few sampled rows only, so dk is exactly their contribution."""
    wl = wk.CHUNKED_PREFILL_128K
    _announce(f"indexer backward 128K prefill, last chunk, two_pass={two_pass}")
    inp = wk.generate(wl, device=DEV)
    L, C = wl.seq_len, wl.chunk
    r0 = L - C
    sl = slice(r0, L)
    prob = dsa.Problem.from_workload(wl, inp, device=DEV, q_rows=sl, q_pos0=r0)
    sub = dict(inp)
    for key in ("q_fp8", "q_scale", "w", "q"):
        sub[key] = inp[key][sl]
    _, idx = _topk(prob, sub)
    rows = [0, 1, 2047, 4095] + [int(x) for x in np.random.default_rng(9).integers(0, C, 4)]
    rows = sorted(set(rows))
    gen = torch.Generator(device="cpu").manual_seed(9)
    grad = torch.zeros(C, wl.topk)
    grad[rows] = torch.randn(len(rows), wl.topk, generator=gen) * 1e-3
    grad = grad.to(DEV)
    dq, dw, dk = _backward(prob, sub, grad, idx, two_pass=two_pass)
    assert torch.isfinite(dq).all() and torch.isfinite(dw).all()
    _check(sub, prob, rows, [r0 + r for r in rows], [0] * len(rows), grad, idx, dq, dw, dk)


def test_backward_two_pass_past_one_scan_window():
    """4600 query rows against the 131072-key prefix in one call: the
    reduction takes a block's tokens 4096 at a time (with 2048 key blocks
    each block has one workgroup).  The gradient is nonzero on sampled rows
    on both sides of the window boundary, so dk is exactly theirs, against
    the oracle; with the gradient on every row, the two-pass dk and the
    atomic one agree to fp32 summation order."""
    wl = wk.CHUNKED_PREFILL_128K
    _announce("indexer backward two-pass, last 4600 rows of the 128K prefill")
    inp = wk.generate(wl, device=DEV)
    L, n = wl.seq_len, 4600
    r0 = L - n
    sl = slice(r0, L)
    prob = dsa.Problem.from_workload(wl, inp, device=DEV, q_rows=sl, q_pos0=r0)
    sub = dict(inp)
    for key in ("q_fp8", "q_scale", "w", "q"):
        sub[key] = inp[key][sl]
    _, idx = _topk(prob, sub)
    rows = [0, 1000, 4095, 4096, 4097, 4599]
    gen = torch.Generator(device="cpu").manual_seed(21)
    grad = torch.zeros(n, wl.topk)
    grad[rows] = torch.randn(len(rows), wl.topk, generator=gen) * 1e-3
    dq, dw, dk = _backward(prob, sub, grad.to(DEV), idx, two_pass=True)
    _check(sub, prob, rows, [r0 + r for r in rows], [0] * len(rows), grad, idx, dq, dw, dk)
    full = (torch.randn(n, wl.topk, generator=gen) * 1e-3).to(DEV)
    _, _, dk_a = _backward(prob, sub, full, idx)
    _, _, dk_t = _backward(prob, sub, full, idx, two_pass=True)
    scale = dk_a.abs().max().item()
    assert scale > 0
    assert (dk_t - dk_a).abs().max().item() <= 1e-5 * scale


def test_backward_two_pass_first_chunk_split_blocks():
    """The first 4096-row chunk of the 128K prefill: 64 key blocks, so each
    block's rows are split over 32 reduction workgroups that add into the
    same dk rows.  Against the atomic path (itself checked against the
    oracle above) on every row, and against the oracle on sampled rows."""
    wl = wk.CHUNKED_PREFILL_128K
    _announce("indexer backward two-pass, first 128K chunk (split blocks)")
    inp = wk.generate(wl, device=DEV)
    C = wl.chunk
    sl = slice(0, C)
    prob = dsa.Problem.from_workload(wl, inp, device=DEV, q_rows=sl, q_pos0=0)
    sub = dict(inp)
    for key in ("q_fp8", "q_scale", "w", "q"):
        sub[key] = inp[key][sl]
    sub["k_fp8"], sub["k_scale"] = inp["k_fp8"][:C], inp["k_scale"][:C]
    _, idx = _topk(prob, sub)
    rows = [0, 5, 2047, 2048, 3000, 4095]
    gen = torch.Generator(device="cpu").manual_seed(23)
    grad = torch.zeros(C, wl.topk)
    grad[rows] = torch.randn(len(rows), wl.topk, generator=gen) * 1e-3
    dq, dw, dk = _backward(prob, sub, grad.to(DEV), idx, two_pass=True)
    _check(sub, prob, rows, rows, [0] * len(rows), grad, idx, dq, dw, dk)
    full = (torch.randn(C, wl.topk, generator=gen) * 1e-3).to(DEV)
    _, _, dk_a = _backward(prob, sub, full, idx)
    _, _, dk_t = _backward(prob, sub, full, idx, two_pass=True)
    scale = dk_a.abs().max().item()
    assert scale > 0
    assert (dk_t - dk_a).abs().max().item() <= 1e-5 * scale


def test_backward_two_pass_keys_shared_by_every_row():
    """Every row of the last 128K chunk selects keys 0..63 (plus 1984 random
    causal keys, ascending): the first 64-key block then holds 4096 x 64
    pairs, 64 of the reduction's 4096-pair batches, and each of those keys'
    runs spans several half-waves.  Sampled rows carry the gradient (dk is
    exactly theirs, against the oracle); with the gradient on every row the
    two-pass dk agrees with the atomic one to fp32 summation order."""
    wl = wk.CHUNKED_PREFILL_128K
    _announce("indexer backward two-pass, keys 0..63 shared by every row")
    inp = wk.generate(wl, device=DEV)
    L, C, k = wl.seq_len, wl.chunk, wl.topk
    r0 = L - C
    sl = slice(r0, L)
    prob = dsa.Problem.from_workload(wl, inp, device=DEV, q_rows=sl, q_pos0=r0)
    sub = dict(inp)
    for key in ("q_fp8", "q_scale", "w", "q"):
        sub[key] = inp[key][sl]
    rng = np.random.default_rng(31)
    idx_np = np.empty((C, k), dtype=np.int32)
    idx_np[:, :64] = np.arange(64)
    for i in range(C):
        idx_np[i, 64:] = np.sort(rng.choice(np.arange(64, r0 + i + 1), size=k - 64, replace=False))
    idx = torch.as_tensor(idx_np, device=DEV)
    rows = [0, 777, 2048, 4095]
    gen = torch.Generator(device="cpu").manual_seed(33)
    grad = torch.zeros(C, k)
    grad[rows] = torch.randn(len(rows), k, generator=gen) * 1e-3
    dq, dw, dk = _backward(prob, sub, grad.to(DEV), idx, two_pass=True)
    _check(sub, prob, rows, [r0 + r for r in rows], [0] * len(rows), grad, idx, dq, dw, dk)
    full = (torch.randn(C, k, generator=gen) * 1e-3).to(DEV)
    _, _, dk_a = _backward(prob, sub, full, idx)
    _, _, dk_t = _backward(prob, sub, full, idx, two_pass=True)
    scale = dk_a.abs().max().item()
    assert scale > 0
    assert (dk_t - dk_a).abs().max().item() <= 1e-5 * scale
