"""dsa_forward_noalloc (dsa_forward with the library's own device scratch as
its workspace) against dsa_forward with a caller workspace, through the C ABI:
identical indices, outputs and lse on two calls in a row, the second with a
smaller problem (the scratch keeps the first call's contents, which the
second must neither need cleared nor leak into its results)."""
import pytest
import torch

from sparse_attention_18_amd import binding as dsa
from sparse_attention_18_amd import workloads as wk

pytestmark = pytest.mark.gpu
DEV = "cuda"

# the 64-sequence decode batch (contexts 8K..128K), then a small prefill
CASES = [("decode_B64_ctx8K_128K", wk.DECODE_B64),
         ("prefill_L1500_k256", wk.PREFILL_4K.scaled(seq_len=1500, topk=256))]


def _run(wl, inp, noalloc):
    prob = dsa.Problem.from_workload(wl, inp, device=DEV)
    T = prob.total_q
    out = torch.full((T, wl.heads, wl.d_latent), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((T, wl.heads), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((T, wl.topk), -7, dtype=torch.int32, device=DEV)
    args = (prob, inp["q_fp8"], inp["q_scale"], inp["w"], inp["k_fp8"], inp["k_scale"], inp["q"],
            inp["kv"], out, lse, idx)
    if noalloc:
        assert dsa.workspace_bytes(prob, dsa.WS_FORWARD) <= dsa.NOALLOC_SCRATCH_BYTES
        dsa.forward_noalloc(*args)
    else:
        ws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_FORWARD), dtype=torch.uint8, device=DEV)
        dsa.forward(*args, workspace=ws)
    torch.cuda.synchronize()
    return idx, out, lse


def test_noalloc_matches_forward_on_two_calls_second_smaller():
    inputs = [wk.generate(wl, device=DEV) for _, wl in CASES]
    refs = []
    for (name, wl), inp in zip(CASES, inputs):
        print(f"[gpu-case] dsa_forward {name}", flush=True)
        refs.append(_run(wl, inp, noalloc=False))
    sizes = [dsa.workspace_bytes(dsa.Problem.from_workload(wl, inp, device=DEV), dsa.WS_FORWARD)
             for (_, wl), inp in zip(CASES, inputs)]
    assert sizes[1] < sizes[0], sizes
    for (name, wl), inp, ref in zip(CASES, inputs, refs):
        print(f"[gpu-case] dsa_forward_noalloc {name}", flush=True)
        got = _run(wl, inp, noalloc=True)
        for a, b, what in zip(got, ref, ("topk_idx", "out", "lse")):
            assert torch.equal(a, b), f"{name}: {what} differs from dsa_forward's"
        assert (got[0] != -7).all() and not torch.isnan(got[1].float()).any()
