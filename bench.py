"""DSA hot-path benchmark on one MI355X.

A step is one pass of the whole path over the 128K-token chunked prefill: 32
chunks of 4096 query rows, each running the lightning indexer, the top-k
selector and the sparse MLA attention against its full causal prefix
(131072 tokens, indexer 64 heads x 128 fp8, k = 2048, 128 heads x 576 bf16).
``value`` is prefill tokens/s over the K timed steps, with every input
already resident in HBM.  The same run also times the decode step (64
sequences, cached contexts uniform in [8K, 128K]) and reports it as
``decode_us_per_step``, the same decode step over paged caches (64-row
blocks, shuffled) as ``decode_paged_us_per_step``, and with the indexer and
the selector fused (dsa_forward_fused) as ``decode_fused_us_per_step``.  ``train_align`` times the
sparse-stage training step: the same 32 chunks, each followed by the indexer
alignment loss over its selected keys (loss and score gradient per row) and
the indexer backward (that gradient carried to dq, dw and dk).

Per-stage durations come from HIP events recorded around each stage call on
the stream the kernels run on.  ``roofline`` covers the dominant stage:
achieved = algorithmic bytes (or flops) / measured time, against MI355X's
published peaks (HBM 8 TB/s, dense FP8 5.0 PFLOP/s, dense bf16 2.5 PFLOP/s).
``cpu_baseline`` is the float64 oracle on a bounded sample of query rows of
the same workload, on the host's cores.

The 4K and 32K prefills (one sequence each, every token a query against its
causal prefix) are timed stage by stage as ``prefill_configs``, with a 1 GiB
read between iterations so that no input is left in the 256 MB MALL; the
decode step is also timed stage by stage (``decode_stages``) and with the
same flush between steps.  ``measured_peaks`` are what the box reaches on
plain work (a device copy, a read-only reduction, large hipBLASLt GEMMs in
bf16 and fp8), and every stage fraction is also given against them
(``frac_measured``).  ``cpu_baseline_configs`` runs the oracle over every row
of the tiny prefill, the 4K prefill and the decode batch, and
``cpu_baseline_single_thread`` a small sample with one BLAS thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode]
                       [--no-train] [--no-cpu-baseline] [--cpu-rows R]
                       [--no-small-prefill] [--only PART] [--stages-json PATH]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from sparse_attention_18_amd import binding as dsa  # noqa: E402
from sparse_attention_18_amd import workloads as wk  # noqa: E402

METRIC = "DSA prefill tokens/s + decode µs/step at 128K ctx; % FP8-MFMA and HBM roofline"
HBM_PEAK = 8.0e12          # B/s
FP8_PEAK = 5.0e15          # dense FLOP/s
BF16_PEAK = 2.5e15


def log(msg):
    print(msg, file=sys.stderr, flush=True)


_KERNEL_SOURCES = {"sparse_attn": ["sparse_attn.hip", "kv_gather.h", "common.h", "launch.h"],
                   "indexer": ["indexer.hip", "common.h", "launch.h"],
                   "topk": ["topk.hip", "common.h", "launch.h"],
                   "align_loss": ["align.hip", "kv_gather.h", "common.h", "launch.h"],
                   "indexer_bwd": ["indexer_bwd.hip", "common.h", "launch.h"]}


def measured_traffic(stage: str):
    """HBM bytes per launch (read + write) from the committed rocprofv3 counter
    summary, or None when the kernel's sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_chunked_prefill_L131072.json")
    try:
        doc = json.load(open(path))
        rec = doc["kernels"][stage]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in _KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, "sparse_attention_18_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != rec.get("source_sha256_16"):
        return None
    return rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]


# ----------------------------------------------------------------- algorithmic work
def indexer_flops(wl, positions):
    """2 * H_I * d_I flop per causal (query, key) pair."""
    pairs = float(np.sum(np.asarray(positions, dtype=np.float64) + 1))
    return 2.0 * wl.idx_heads * wl.idx_dim * pairs


def topk_bytes(wl, positions):
    """4 B read per causal candidate + 4 B written per index slot."""
    n = np.asarray(positions, dtype=np.float64) + 1
    return 4.0 * float(n.sum()) + 4.0 * wl.topk * len(n)


def attn_bytes(wl, positions):
    """Per selected pair: one latent KV row (576 bf16 = 1152 B) + its 4 B
    index; per token: q (H x 576 bf16) in, out (H x 512 bf16) out."""
    m = np.minimum(np.asarray(positions, dtype=np.float64) + 1, wl.topk)
    per_tok = wl.heads * wl.d_qk * 2 + wl.heads * wl.d_latent * 2
    return float(m.sum()) * (wl.d_qk * 2 + 4) + per_tok * len(m)


def attn_flops(wl, positions):
    m = np.minimum(np.asarray(positions, dtype=np.float64) + 1, wl.topk)
    return float(m.sum()) * 2.0 * wl.heads * (wl.d_qk + wl.d_latent)


def align_bytes(wl, positions):
    """Alignment loss, per selected pair: the latent KV row (1152 B), its index,
    its score and its gradient (4 B each); per token: q (H x 576 bf16), lse
    (H floats) and the loss."""
    m = np.minimum(np.asarray(positions, dtype=np.float64) + 1, wl.topk)
    per_tok = wl.heads * wl.d_qk * 2 + wl.heads * 4 + 4
    return float(m.sum()) * (wl.d_qk * 2 + 12) + per_tok * len(m)


def indexer_bwd_bytes(wl, positions):
    """Indexer backward, read or written once: per selected pair the key row,
    its scale and the score gradient (128 + 4 + 4 B); per query q8, w, q_scale
    in and dq (fp32), dw out; dk (fp32) once per key."""
    m = np.minimum(np.asarray(positions, dtype=np.float64) + 1, wl.topk)
    per_tok = wl.idx_heads * wl.idx_dim * (1 + 4) + wl.idx_heads * 4 * 2 + 4
    return float(m.sum()) * (wl.idx_dim + 8) + per_tok * len(m) + 4.0 * wl.idx_dim * len(m)


def indexer_bwd_flops(wl, positions):
    """z (2 H_I d_I), dq and dk (2 H_I d_I each) per selected pair."""
    m = np.minimum(np.asarray(positions, dtype=np.float64) + 1, wl.topk)
    return float(m.sum()) * 6.0 * wl.idx_heads * wl.idx_dim


def align_flops(wl, positions):
    m = np.minimum(np.asarray(positions, dtype=np.float64) + 1, wl.topk)
    return float(m.sum()) * 2.0 * wl.heads * wl.d_qk


def indexer_decode_bytes(wl, positions):
    """Decode indexer (HBM-bound): per cached key its FP8 row and scale read
    once and its fp32 score written (d_I + 4 + 4 B)."""
    n = np.asarray(positions, dtype=np.float64) + 1
    return float(n.sum()) * (wl.idx_dim + 8)


# ----------------------------------------------------------------- measured peaks
def _median_seconds(fn, n=10, warm=3):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(n):
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts)) * 1e-3


def measured_peaks(dev):
    """What this machine reaches on plain work: a 2 GiB device copy (read + write
    bytes), a read-only reduction over it, and 8192^3 GEMMs through torch
    (hipBLASLt) in bf16 and fp8 e4m3.  Context for the spec peaks, not a
    replacement: each stage fraction is reported against both."""
    res = {}
    src = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    nbytes = src.numel() * 4
    res["hbm_copy_GBps"] = round(2 * nbytes / _median_seconds(lambda: dst.copy_(src)) / 1e9, 1)
    res["hbm_read_GBps"] = round(nbytes / _median_seconds(lambda: src.sum()) / 1e9, 1)
    del src, dst
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    res["bf16_gemm_TFLOPs"] = round(2 * n ** 3 / _median_seconds(lambda: torch.mm(a, b)) / 1e12, 1)
    try:
        a8 = a.to(torch.float8_e4m3fn)
        b8 = b.to(torch.float8_e4m3fn).t()          # column-major right operand
        one = torch.ones((), device=dev)
        t = _median_seconds(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one,
                                                     out_dtype=torch.bfloat16))
        res["fp8_gemm_TFLOPs"] = round(2 * n ** 3 / t / 1e12, 1)
    except Exception as e:  # pragma: no cover - depends on the torch build
        log(f"[bench] fp8 GEMM probe unavailable: {e}")
        res["fp8_gemm_TFLOPs"] = None
    res["how"] = ("2 GiB torch copy_ (read + write bytes) and sum (read bytes); 8192^3 torch.mm "
                  "(bf16) and torch._scaled_mm (fp8 e4m3, bf16 out); medians of 10")
    return res


_SPEC = {"hbm": (HBM_PEAK, "GB/s", 1e9), "mfma": (FP8_PEAK, "TFLOP/s", 1e12),
         "mfma_bf16": (BF16_PEAK, "TFLOP/s", 1e12)}


def _measured_peak(bound, peaks):
    if not peaks:
        return None
    if bound == "hbm":
        return max(peaks["hbm_copy_GBps"], peaks["hbm_read_GBps"]) * 1e9
    v = peaks.get("bf16_gemm_TFLOPs" if bound == "mfma_bf16" else "fp8_gemm_TFLOPs")
    return v * 1e12 if v else None


def stage_entry(ms, launches, bound, amount, peaks=None, bf16_flops=None):
    """One stage's record: time, algorithmic rate, and its fraction of the spec
    peak (``frac``) and of the box's measured peak (``frac_measured``)."""
    peak, unit, scale = _SPEC[bound]
    t = ms * 1e-3
    rate = amount / t
    e = {"ms_per_step": round(ms, 4), "launches_per_step": launches,
         "avg_launch_us": round(ms / launches * 1e3, 1), "bound": bound,
         "achieved": round(rate / scale, 1), "peak": round(peak / scale, 1), "unit": unit,
         "frac": round(rate / peak, 4)}
    mp = _measured_peak(bound, peaks)
    if mp:
        e["frac_measured"] = round(rate / mp, 4)
    if bf16_flops is not None:
        e["bf16_tflops"] = round(bf16_flops / t / 1e12, 1)
        e["bf16_mfma_frac"] = round(bf16_flops / t / BF16_PEAK, 4)
        if peaks and peaks.get("bf16_gemm_TFLOPs"):
            e["bf16_frac_measured"] = round(bf16_flops / t / (peaks["bf16_gemm_TFLOPs"] * 1e12), 4)
    return e


# ----------------------------------------------------------------- prefill step
class ChunkedPrefill:
    def __init__(self, wl, dev):
        self.wl = wl
        t0 = time.time()
        self.inp = wk.generate(wl, device=dev)
        torch.cuda.synchronize()
        log(f"[bench] generated {wl.name} inputs on {dev} in {time.time() - t0:.1f}s")
        L, C = wl.seq_len, wl.chunk
        self.chunks = []
        for r0, sl in wk.chunk_views(self.inp, C):
            prob = dsa.Problem.from_workload(wl, self.inp, device=dev, q_rows=sl, q_pos0=r0)
            self.chunks.append((r0, sl, prob))
        self.ld = self.chunks[-1][2].ld_scores()
        self.scores = torch.empty(C, self.ld, dtype=torch.float32, device=dev)
        self.idx = torch.empty(L, wl.topk, dtype=torch.int32, device=dev)
        self.out = torch.empty(L, wl.heads, wl.d_latent, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(L, wl.heads, dtype=torch.float32, device=dev)
        self.positions = np.arange(L)
        self.n_stage_events = 0

    def step(self, events=None):
        inp, wl = self.inp, self.wl
        for ci, (r0, sl, prob) in enumerate(self.chunks):
            rows = sl.stop - sl.start
            scores = self.scores[:rows]
            if events is not None:
                events[ci][0].record()
            dsa.indexer_scores(prob, inp["q_fp8"][sl], inp["q_scale"][sl], inp["w"][sl],
                               inp["k_fp8"][: sl.stop], inp["k_scale"][: sl.stop],
                               scores, self.ld)
            if events is not None:
                events[ci][1].record()
            dsa.topk(prob, scores, self.idx[sl], ld=self.ld)
            if events is not None:
                events[ci][2].record()
            dsa.sparse_attn(prob, inp["q"][sl], inp["kv"][: sl.stop], self.idx[sl],
                            self.out[sl], self.lse[sl])
            if events is not None:
                events[ci][3].record()

    def train_step(self, events=None):
        """The forward chunks, each followed by the indexer alignment loss over
        its selected keys (while the chunk's scores are still in place)."""
        inp, wl = self.inp, self.wl
        if not hasattr(self, "grad"):
            dev = self.scores.device
            self.grad = torch.empty(wl.chunk, wl.topk, dtype=torch.float32, device=dev)
            self.loss = torch.empty(wl.seq_len, dtype=torch.float32, device=dev)
            self.dq = torch.empty(wl.chunk, wl.idx_heads, wl.idx_dim, dtype=torch.float32, device=dev)
            self.dw = torch.empty(wl.chunk, wl.idx_heads, dtype=torch.float32, device=dev)
            self.dk = torch.zeros(wl.seq_len, wl.idx_dim, dtype=torch.float32, device=dev)
            # the indexer backward's two-pass dk (the largest chunk's size serves all)
            n = max(dsa.workspace_bytes(prob, dsa.WS_INDEXER_BWD) for _, _, prob in self.chunks)
            self.bwd_ws = torch.empty(n, dtype=torch.uint8, device=dev)
        self.dk.zero_()
        for ci, (r0, sl, prob) in enumerate(self.chunks):
            rows = sl.stop - sl.start
            scores = self.scores[:rows]
            dsa.indexer_scores(prob, inp["q_fp8"][sl], inp["q_scale"][sl], inp["w"][sl],
                               inp["k_fp8"][: sl.stop], inp["k_scale"][: sl.stop],
                               scores, self.ld)
            dsa.topk(prob, scores, self.idx[sl], ld=self.ld)
            dsa.sparse_attn(prob, inp["q"][sl], inp["kv"][: sl.stop], self.idx[sl],
                            self.out[sl], self.lse[sl])
            if events is not None:
                events[ci][0].record()
            dsa.indexer_align_loss(prob, inp["q"][sl], inp["kv"][: sl.stop], self.lse[sl], scores,
                                   self.loss[sl], self.grad[:rows], idx=self.idx[sl], ld=self.ld)
            if events is not None:
                events[ci][1].record()
            dsa.indexer_backward(prob, inp["q_fp8"][sl], inp["q_scale"][sl], inp["w"][sl],
                                 inp["k_fp8"][: sl.stop], inp["k_scale"][: sl.stop], self.grad[:rows],
                                 self.dq[:rows], self.dw[:rows], self.dk[: sl.stop], idx=self.idx[sl],
                                 workspace=self.bwd_ws)
            if events is not None:
                events[ci][2].record()


def run_prefill(args, dev, peaks=None):
    wl = wk.CHUNKED_PREFILL_128K
    bench = ChunkedPrefill(wl, dev)
    for i in range(args.warmup):
        bench.step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")
    nch = len(bench.chunks)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nch)]
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        bench.step(evs[s])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    log(f"[bench] {args.steps} timed steps: {gpu_ms:.1f} ms (events), {wall * 1e3:.1f} ms (wall)")
    stage_ms = np.zeros(3)
    per_chunk = np.zeros((nch, 3))
    for s in range(args.steps):
        for c in range(nch):
            e = evs[s][c]
            for j in range(3):
                dt = e[j].elapsed_time(e[j + 1])
                stage_ms[j] += dt
                per_chunk[c, j] += dt
    stage_ms /= args.steps
    per_chunk /= args.steps
    pos = bench.positions
    stages = {
        "indexer": stage_entry(stage_ms[0], nch, "mfma", indexer_flops(wl, pos), peaks),
        "topk": stage_entry(stage_ms[1], nch, "hbm", topk_bytes(wl, pos), peaks),
        "sparse_attn": stage_entry(stage_ms[2], nch, "hbm", attn_bytes(wl, pos), peaks,
                                   bf16_flops=attn_flops(wl, pos)),
    }
    ms_per_step = gpu_ms / args.steps
    value = wl.seq_len / (ms_per_step * 1e-3)
    return bench, wl, value, ms_per_step, stages, per_chunk


class MallFlush:
    """A 1 GiB buffer read between timed iterations: four times the 256 MB
    MALL, so no input of the previous iteration is still cached there.  A
    read, not a write: written lines would be written back to HBM while the
    next timed kernel runs, and that kernel would pay for them."""

    def __init__(self, dev):
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def __call__(self):
        torch.sum(self.buf)


def run_prefill_single(wl, dev, flush, peaks=None, iters=10, warmup=2):
    """One prefill sequence, every token a query against its causal prefix:
    indexer, top-k and attention through the three stage calls, each stage
    bracketed by events, the MALL flushed before every iteration.  Returns
    the medians over the iterations and the inputs (for the CPU baseline)."""
    t0 = time.time()
    inp = wk.generate(wl, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] generated {wl.name} inputs in {time.time() - t0:.1f}s")
    prob = dsa.Problem.from_workload(wl, inp, device=dev)
    L, ld = wl.seq_len, prob.ld_scores()
    scores = torch.empty(L, ld, dtype=torch.float32, device=dev)
    idx = torch.empty(L, wl.topk, dtype=torch.int32, device=dev)
    out = torch.empty(L, wl.heads, wl.d_latent, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(L, wl.heads, dtype=torch.float32, device=dev)
    nt, na = dsa.workspace_bytes(prob, dsa.WS_TOPK), dsa.workspace_bytes(prob, dsa.WS_ATTN)
    tws = torch.empty(nt, dtype=torch.uint8, device=dev) if nt else None
    aws = torch.empty(na, dtype=torch.uint8, device=dev) if na else None

    def run(ev):
        ev[0].record()
        dsa.indexer_scores(prob, inp["q_fp8"], inp["q_scale"], inp["w"], inp["k_fp8"], inp["k_scale"],
                           scores, ld)
        ev[1].record()
        dsa.topk(prob, scores, idx, ld=ld, workspace=tws)
        ev[2].record()
        dsa.sparse_attn(prob, inp["q"], inp["kv"], idx, out, lse, workspace=aws)
        ev[3].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(warmup + iters)]
    for i in range(warmup + iters):
        flush()
        run(evs[i])
    torch.cuda.synchronize()
    t = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs[warmup:]])
    med = np.median(t, axis=0)
    total = float(np.median(t.sum(axis=1)))
    pos = np.arange(L)
    stages = {"indexer": stage_entry(med[0], 1, "mfma", indexer_flops(wl, pos), peaks),
              "topk": stage_entry(med[1], 1, "hbm", topk_bytes(wl, pos), peaks),
              "sparse_attn": stage_entry(med[2], 1, "hbm", attn_bytes(wl, pos), peaks,
                                         bf16_flops=attn_flops(wl, pos))}
    log(f"[bench] {wl.name}: {total:.3f} ms per pass (indexer {med[0]:.3f}, top-k {med[1]:.3f}, "
        f"attention {med[2]:.3f} ms), MALL flushed between passes")
    res = {"workload": wl.name, "tokens_per_s": round(L / (total * 1e-3), 1), "ms": round(total, 4),
           "iters": iters, "mall_flushed": True, "stages": stages}
    del scores, out, lse, tws, aws
    res["prefill_mode_attention"] = run_prefill_mode(wl, dev, flush, prob, idx, med[2], peaks, iters, warmup)
    return res, inp, idx


def run_prefill_mode(wl, dev, flush, prob, idx, absorbed_ms, peaks, iters, warmup):
    """The same selection through the prefill-mode attention (per-head keys of
    128 + 64 and values of 128, the selection as a mask over dense key tiles),
    on seeded inputs of that form.  Its roofline is bf16 MFMA on the dense work
    it does (every causal pair of the tiles it visits, here all of them); the
    flops of the selected pairs alone are reported beside it."""
    L, H = wl.seq_len, wl.heads
    inp = wk.mha_prefill_inputs(L, L, H, seed=wl.seed + 100, device=dev)
    out = torch.empty(L, H, wk.MHA_V, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(L, H, dtype=torch.float32, device=dev)
    ws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_ATTN_PREFILL), dtype=torch.uint8, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(warmup + iters)]
    for i in range(warmup + iters):
        flush()
        evs[i][0].record()
        dsa.sparse_attn_prefill(prob, inp["q"], inp["k_nope"], inp["k_rope"], inp["v"], idx, out, lse, ws)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs[warmup:]]))
    per_pair = 2 * H * (wk.MHA_NOPE + wk.MHA_ROPE + wk.MHA_V)
    causal = L * (L + 1) // 2
    selected = int((idx >= 0).sum())
    e = stage_entry(ms, 1, "mfma_bf16", per_pair * causal, peaks)
    e["selected_pair_tflops"] = round(per_pair * selected / (ms * 1e-3) / 1e12, 1)
    e["vs_absorbed_form"] = round(absorbed_ms / ms, 3)
    log(f"[bench] {wl.name}: prefill-mode attention {ms:.3f} ms ({e['achieved']} TFLOP/s on the causal "
        f"pairs, {e['frac']:.3f} of bf16 peak; absorbed form {absorbed_ms:.3f} ms)")
    del inp, out, lse, ws
    return e


def run_train(bench, steps=2):
    """Sparse-stage training step: forward chunks plus the alignment loss."""
    wl = bench.wl
    bench.train_step()
    torch.cuda.synchronize()
    nch = len(bench.chunks)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nch)]
           for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(steps):
        bench.train_step(evs[s])
    end.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / steps
    loss_ms = sum(e[0].elapsed_time(e[1]) for st in evs for e in st) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for st in evs for e in st) / steps
    pos = bench.positions
    t = loss_ms * 1e-3
    rate = align_bytes(wl, pos) / t
    tb = bwd_ms * 1e-3
    brate = indexer_bwd_bytes(wl, pos) / tb
    log(f"[bench] training step {step_ms:.1f} ms, alignment loss {loss_ms:.2f} ms, "
        f"indexer backward {bwd_ms:.2f} ms")
    bwd = {"ms_per_step": round(bwd_ms, 3), "launches_per_step": nch,
           "avg_launch_us": round(bwd_ms / nch * 1e3, 1), "bound": "hbm",
           "achieved": round(brate / 1e9, 1), "peak": round(HBM_PEAK / 1e9, 1), "unit": "GB/s",
           "frac": round(brate / HBM_PEAK, 4),
           "tflops": round(indexer_bwd_flops(wl, pos) / tb / 1e12, 1),
           "traffic": measured_traffic("indexer_bwd")}
    return {"ms_per_step": round(loss_ms, 3), "launches_per_step": nch,
            "avg_launch_us": round(loss_ms / nch * 1e3, 1), "bound": "hbm",
            "achieved": round(rate / 1e9, 1), "peak": round(HBM_PEAK / 1e9, 1), "unit": "GB/s",
            "frac": round(rate / HBM_PEAK, 4),
            "bf16_tflops": round(align_flops(wl, pos) / t / 1e12, 1),
            "traffic": measured_traffic("align_loss"),
            "train_step_ms": round(step_ms, 3),
            "train_tokens_per_s": round(wl.seq_len / (step_ms * 1e-3), 1),
            "indexer_backward": bwd,
            "steps": steps}


def train_cpu_baseline(bench, wl, rows_n=512, batch=32):
    """The float64 oracle's alignment loss and indexer backward on sampled rows
    of the last chunk, on the GPU's own scores, indices and score gradient.
    Rows are copied to the host a batch at a time (untimed); only the oracle
    calls are timed."""
    import oracle
    threads = _blas_threads()
    inp, L, C = bench.inp, wl.seq_len, wl.chunk
    r0 = L - C
    rows_all = np.linspace(0, C - 1, rows_n).astype(np.int64)
    dt = 0.0
    for b0 in range(0, rows_n, batch):
        rows = rows_all[b0:b0 + batch]
        idx = bench.idx[r0 + rows].cpu().numpy()
        sc = bench.scores[rows].cpu().double().numpy()      # the last chunk's scores
        g = bench.grad[rows].cpu().double().numpy()
        cases = []
        for i, r in enumerate(rows):
            keys = idx[i][idx[i] >= 0].astype(np.int64)
            at = torch.as_tensor(keys)
            cases.append(dict(
                q=inp["q"][r0 + r].cpu().double().numpy(), kv=inp["kv"][at].cpu().double().numpy(),
                qd=oracle.dequantize(inp["q_fp8"][r0 + r:r0 + r + 1].cpu().numpy(),
                                     inp["q_scale"][r0 + r:r0 + r + 1].cpu().numpy())[0],
                w=inp["w"][r0 + r].cpu().double().numpy(),
                kd=oracle.dequantize(inp["k_fp8"][at].cpu().numpy(), inp["k_scale"][at].cpu().numpy()),
                s=sc[i][keys], g=g[i][: keys.size], pos=r0 + int(r), m=keys.size))
        t0 = time.perf_counter()
        for c in cases:
            local = np.arange(c["m"])[None]
            oracle.alignment_loss_rows(c["q"][None], c["kv"], [c["s"]], [c["pos"]], wl.softmax_scale,
                                       idx=local)
            oracle.indexer_backward_rows(c["qd"][None], c["w"][None], c["kd"], [c["pos"]], [c["g"]],
                                         idx=local)
        dt += time.perf_counter() - t0
    log(f"[bench] training cpu baseline: {dt:.1f}s for {rows_n} rows")
    return {"value": round(rows_n / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows_n} rows of the last 4096-row chunk, 2048 selected keys each "
                      f"(alignment loss and indexer backward in float64 per row, on the GPU's "
                      f"scores, indices and score gradient; every row of the step costs the same "
                      f"except the first 2048, so the rate stands for the whole step)",
            "seconds": round(dt, 2)}


def run_decode(args, dev):
    wl = wk.DECODE_B64
    t0 = time.time()
    inp = wk.generate(wl, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] generated {wl.name} inputs in {time.time() - t0:.1f}s "
        f"(total cached keys {inp['kv_offsets'][-1]})")
    prob = dsa.Problem.from_workload(wl, inp, device=dev)
    B = wl.decode_batch
    out = torch.empty(B, wl.heads, wl.d_latent, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, wl.heads, dtype=torch.float32, device=dev)
    idx = torch.empty(B, wl.topk, dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_FORWARD), dtype=torch.uint8, device=dev)

    def step():
        dsa.forward(prob, inp["q_fp8"], inp["q_scale"], inp["w"], inp["k_fp8"], inp["k_scale"],
                    inp["q"], inp["kv"], out, lse, idx, ws)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    n = 20
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        step()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n
    log(f"[bench] decode step {us:.1f} us")

    # The same step over paged caches (64-row blocks, shuffled).
    table, nblocks, kc, ksc, kvc = wk.paged_caches(inp, 64, seed=1, device=dev)
    pg = dsa.PagedKV(table, 64, nblocks, device=dev)

    def step_paged():
        dsa.forward_paged(prob, pg, inp["q_fp8"], inp["q_scale"], inp["w"], kc, ksc, inp["q"], kvc,
                          out, lse, idx, ws)

    for _ in range(3):
        step_paged()
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        step_paged()
    b.record()
    torch.cuda.synchronize()
    us_paged = a.elapsed_time(b) * 1e3 / n
    log(f"[bench] decode step over paged caches {us_paged:.1f} us")
    del kc, ksc, kvc

    # The same step with the indexer and the selector fused (dsa_forward_fused).
    fws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_FORWARD_FUSED), dtype=torch.uint8, device=dev)

    def step_fused():
        dsa.forward_fused(prob, inp["q_fp8"], inp["q_scale"], inp["w"], inp["k_fp8"], inp["k_scale"],
                          inp["q"], inp["kv"], out, lse, idx, fws)

    for _ in range(3):
        step_fused()
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        step_fused()
    b.record()
    torch.cuda.synchronize()
    us_fused = a.elapsed_time(b) * 1e3 / n
    log(f"[bench] decode step with the fused indexer and top-k {us_fused:.1f} us")
    del fws
    return us, us_paged, us_fused, inp


def run_decode_stages(inp, dev, flush, peaks=None, iters=20, warmup=3):
    """The decode step stage by stage (indexer, top-k, attention through the
    stage calls, each bracketed by events) and whole (dsa_forward), each
    iteration after a MALL flush, as a decode step that follows other work
    would run.  Medians."""
    wl = wk.DECODE_B64
    prob = dsa.Problem.from_workload(wl, inp, device=dev)
    B, ld = wl.decode_batch, prob.ld_scores()
    scores = torch.empty(B, ld, dtype=torch.float32, device=dev)
    out = torch.empty(B, wl.heads, wl.d_latent, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, wl.heads, dtype=torch.float32, device=dev)
    idx = torch.empty(B, wl.topk, dtype=torch.int32, device=dev)
    nt, na = dsa.workspace_bytes(prob, dsa.WS_TOPK), dsa.workspace_bytes(prob, dsa.WS_ATTN)
    tws = torch.empty(nt, dtype=torch.uint8, device=dev) if nt else None
    aws = torch.empty(na, dtype=torch.uint8, device=dev) if na else None
    fws = torch.empty(dsa.workspace_bytes(prob, dsa.WS_FORWARD), dtype=torch.uint8, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(warmup + iters)]
    for i in range(warmup + iters):
        e = ev[i]
        flush()
        e[0].record()
        dsa.indexer_scores(prob, inp["q_fp8"], inp["q_scale"], inp["w"], inp["k_fp8"], inp["k_scale"],
                           scores, ld)
        e[1].record()
        dsa.topk(prob, scores, idx, ld=ld, workspace=tws)
        e[2].record()
        dsa.sparse_attn(prob, inp["q"], inp["kv"], idx, out, lse, workspace=aws)
        e[3].record()
        flush()
        e[4].record()
        dsa.forward(prob, inp["q_fp8"], inp["q_scale"], inp["w"], inp["k_fp8"], inp["k_scale"],
                    inp["q"], inp["kv"], out, lse, idx, fws)
        e[5].record()
    torch.cuda.synchronize()
    t = np.array([[e[j].elapsed_time(e[j + 1]) for j in (0, 1, 2, 4)] for e in ev[warmup:]])
    med = np.median(t, axis=0)
    pos = np.asarray(inp["q_pos0"], dtype=np.int64)
    stages = {"indexer": stage_entry(med[0], 1, "hbm", indexer_decode_bytes(wl, pos), peaks),
              "topk": stage_entry(med[1], 1, "hbm", topk_bytes(wl, pos), peaks),
              "sparse_attn": stage_entry(med[2], 1, "hbm", attn_bytes(wl, pos), peaks,
                                         bf16_flops=attn_flops(wl, pos))}
    for v in stages.values():
        v["us"] = round(v.pop("ms_per_step") * 1e3, 1)
        v.pop("launches_per_step")
        v.pop("avg_launch_us")
    ideal = (indexer_decode_bytes(wl, pos) + topk_bytes(wl, pos) + attn_bytes(wl, pos)) / HBM_PEAK
    log(f"[bench] decode stages after a MALL flush: indexer {med[0] * 1e3:.1f} us, top-k "
        f"{med[1] * 1e3:.1f} us, attention {med[2] * 1e3:.1f} us; dsa_forward {med[3] * 1e3:.1f} us")
    return {"forward_us_mall_flushed": round(med[3] * 1e3, 1), "stages": stages,
            "ideal_us_at_hbm_peak": round(ideal * 1e6, 1), "iters": iters}


def cpu_baseline(bench, wl, rows_n):
    """The float64 oracle on a stratified sample of query rows of the prefill."""
    import oracle
    threads = _blas_threads()
    inp = bench.inp
    L = wl.seq_len
    rng = np.random.default_rng(wl.seed)
    rows = np.unique(np.concatenate([np.linspace(0, L - 1, rows_n).astype(np.int64),
                                     rng.integers(0, L, 4)]))
    t_copy = time.time()
    kd_all = oracle.dequantize(inp["k_fp8"].cpu().numpy(), inp["k_scale"].cpu().numpy())
    kv_all = inp["kv"].cpu().double().numpy()
    qd = oracle.dequantize(inp["q_fp8"][rows].cpu().numpy(), inp["q_scale"][rows].cpu().numpy())
    w = inp["w"][rows].cpu().double().numpy()
    qa = inp["q"][rows].cpu().double().numpy()
    log(f"[bench] cpu baseline: copied inputs in {time.time() - t_copy:.1f}s; "
        f"{len(rows)} rows, {threads} threads")
    t0 = time.perf_counter()
    oracle.forward_rows(qd, w, kd_all, rows, qa, kv_all, wl.topk, wl.softmax_scale, wl.d_latent)
    dt = time.perf_counter() - t0
    log(f"[bench] cpu baseline: {dt:.1f}s for {len(rows)} rows")
    # rows differ in cost (causal); scale the sample's mean cost to all L rows
    frac = float(np.sum(rows + 1)) / float(np.sum(np.arange(1, L + 1))) * L / len(rows)
    tok_s = len(rows) * frac / dt if dt > 0 else float("nan")
    return {"value": round(tok_s, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} query rows spread evenly over the 131072-token sequence "
                      f"(indexer, top-k and attention in float64 per row; the rate is scaled "
                      f"to the full sequence by the sampled rows' causal-length share)",
            "seconds": round(dt, 2)}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def _oracle_prefill_rows(inp, wl, rows, block=512):
    """Time the oracle's forward over packed prefill rows (host copies made per
    block, untimed); returns seconds."""
    import oracle
    kd = oracle.dequantize(inp["k_fp8"].cpu().numpy(), inp["k_scale"].cpu().numpy())
    kv = inp["kv"].cpu().double().numpy()
    dt = 0.0
    for b0 in range(0, len(rows), block):
        r = rows[b0:b0 + block]
        at = torch.as_tensor(r)
        qd = oracle.dequantize(inp["q_fp8"][at].cpu().numpy(), inp["q_scale"][at].cpu().numpy())
        w = inp["w"][at].cpu().double().numpy()
        qa = inp["q"][at].cpu().double().numpy()
        t0 = time.perf_counter()
        oracle.forward_rows(qd, w, kd, r, qa, kv, wl.topk, wl.softmax_scale, wl.d_latent)
        dt += time.perf_counter() - t0
    return dt


def cpu_baseline_configs(dev, prefill_4k_inp=None, decode_inp=None):
    """The oracle over every row of the tiny prefill and the 4K prefill, and
    every sequence of the decode batch, on the inputs the GPU ran."""
    import oracle
    res = {}
    for wl, inp in ((wk.TINY_PREFILL, None), (wk.PREFILL_4K, prefill_4k_inp)):
        if inp is None:
            inp = wk.generate(wl, device=dev)
        L = wl.seq_len
        dt = _oracle_prefill_rows(inp, wl, np.arange(L))
        res[wl.name] = {"value": round(L / dt, 2), "unit": "tokens/s", "seconds": round(dt, 2),
                        "rows": L, "sample": "every query row"}
        log(f"[bench] cpu baseline {wl.name}: {dt:.1f}s for all {L} rows")
    if decode_inp is not None:
        wl, inp = wk.DECODE_B64, decode_inp
        dt = 0.0
        for b in range(wl.decode_batch):
            k0, k1 = inp["kv_offsets"][b], inp["kv_offsets"][b + 1]
            kd = oracle.dequantize(inp["k_fp8"][k0:k1].cpu().numpy(), inp["k_scale"][k0:k1].cpu().numpy())
            kv = inp["kv"][k0:k1].cpu().double().numpy()
            qd = oracle.dequantize(inp["q_fp8"][b:b + 1].cpu().numpy(), inp["q_scale"][b:b + 1].cpu().numpy())
            w = inp["w"][b:b + 1].cpu().double().numpy()
            qa = inp["q"][b:b + 1].cpu().double().numpy()
            t0 = time.perf_counter()
            oracle.forward_rows(qd, w, kd, [k1 - k0 - 1], qa, kv, wl.topk, wl.softmax_scale, wl.d_latent)
            dt += time.perf_counter() - t0
        res[wl.name] = {"value": round(dt * 1e6, 1), "unit": "us/step", "seconds": round(dt, 2),
                        "rows": wl.decode_batch, "sample": "every sequence of the batch"}
        log(f"[bench] cpu baseline {wl.name}: {dt:.1f}s for all {wl.decode_batch} sequences")
    return res


def cpu_baseline_single_thread(bench, wl, rows_n=48):
    """The oracle on a small sample of the 128K prefill's rows with one BLAS
    thread, scaled to tokens/s like the headline baseline."""
    from threadpoolctl import threadpool_limits
    L = wl.seq_len
    rows = np.linspace(0, L - 1, rows_n).astype(np.int64)
    with threadpool_limits(limits=1):
        dt = _oracle_prefill_rows(bench.inp, wl, rows)
    frac = float(np.sum(rows + 1)) / float(np.sum(np.arange(1, L + 1))) * L / len(rows)
    log(f"[bench] single-thread cpu baseline: {dt:.1f}s for {rows_n} rows")
    return {"value": round(len(rows) * frac / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows_n} query rows spread evenly over the 131072-token sequence, one BLAS "
                      f"thread, scaled like cpu_baseline", "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-train", action="store_true", help="skip the alignment-loss training step")
    ap.add_argument("--no-small-prefill", action="store_true", help="skip the 4K and 32K prefills")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--only", choices=("prefill", "train", "decode", "small_prefill"), default=None,
                    help="run only this part (for profiling runs; the headline fields are then "
                         "null unless the part is the 128K prefill)")
    ap.add_argument("--stages-json", default=None, help="also write per-chunk stage times here")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build runs the DSA path on a single "
              f"MI355X and has no multi-GPU mode (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
        # the scale from counter units to bytes for the kernels' counters.
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "copies": 3}))
        return
    dsa.load_library()
    only = args.only
    do = {"prefill": only in (None, "prefill", "train"),
          "train": (only is None and not args.no_train) or only == "train",
          "decode": (only is None and not args.no_decode) or only == "decode",
          "small_prefill": (only is None and not args.no_small_prefill) or only == "small_prefill"}
    cpu_on = only is None and not args.no_cpu_baseline
    peaks = measured_peaks(dev) if only is None else None
    if peaks:
        log(f"[bench] measured peaks: {peaks}")
    flush = MallFlush(dev)
    wl = wk.CHUNKED_PREFILL_128K
    bench = value = ms_per_step = stages = roofline = topk_plus_attn = None
    if do["prefill"]:
        bench, wl, value, ms_per_step, stages, per_chunk = run_prefill(args, dev, peaks)
        dominant = max(stages, key=lambda s: stages[s]["ms_per_step"])
        d = stages[dominant]
        roofline = {"bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"],
                    "unit": d["unit"], "frac": d["frac"], "traffic": measured_traffic(dominant),
                    "kernel": dominant,
                    "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE)"}
        if "frac_measured" in d:
            roofline["frac_measured"] = d["frac_measured"]
        # top-k and sparse attention together: their algorithmic bytes over
        # their summed time (the two HBM-bound stages of the step)
        both_ms = stages["topk"]["ms_per_step"] + stages["sparse_attn"]["ms_per_step"]
        topk_plus_attn = stage_entry(both_ms, stages["topk"]["launches_per_step"] * 2, "hbm",
                                     topk_bytes(wl, bench.positions) + attn_bytes(wl, bench.positions),
                                     peaks)
        if args.stages_json:
            with open(args.stages_json, "w") as f:
                json.dump({"stages": stages, "per_chunk_ms": per_chunk.tolist()}, f, indent=1)
    train = None
    if do["train"]:
        train = run_train(bench)
        if cpu_on:
            train["cpu_baseline"] = train_cpu_baseline(bench, wl)
    decode_us = decode_paged_us = decode_fused_us = decode_stages = decode_inp = None
    if do["decode"]:
        decode_us, decode_paged_us, decode_fused_us, decode_inp = run_decode(args, dev)
        decode_stages = run_decode_stages(decode_inp, dev, flush, peaks)
    prefill_configs = {}
    p4k_inp = None
    if do["small_prefill"]:
        for swl in (wk.PREFILL_4K, wk.PREFILL_32K_BOOSTED):
            res, inp, _ = run_prefill_single(swl, dev, flush, peaks)
            prefill_configs[swl.name] = res
            if swl is wk.PREFILL_4K:
                p4k_inp = inp
            del inp
            torch.cuda.empty_cache()
    cpu = cpu1 = cpu_cfgs = None
    if cpu_on and bench is not None:
        cpu = cpu_baseline(bench, wl, args.cpu_rows)
        cpu1 = cpu_baseline_single_thread(bench, wl)
        cpu_cfgs = cpu_baseline_configs(dev, p4k_inp, decode_inp)
    line = {
        "metric": METRIC, "value": None if value is None else round(value, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None if ms_per_step is None else round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3+bf16", "data": "synthetic",
        "config": {"workload": wl.name, "seq_len": wl.seq_len, "chunk": wl.chunk,
                   "topk": wl.topk, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim,
                   "heads": wl.heads, "d_qk": wl.d_qk, "d_latent": wl.d_latent,
                   "parallelism": "single GPU"},
        "decode_us_per_step": None if decode_us is None else round(decode_us, 1),
        "decode_paged_us_per_step": None if decode_paged_us is None else round(decode_paged_us, 1),
        "decode_fused_us_per_step": None if decode_fused_us is None else round(decode_fused_us, 1),
        "decode_config": {"workload": wk.DECODE_B64.name, "batch": 64,
                          "ctx": [wk.DECODE_B64.ctx_min, wk.DECODE_B64.ctx_max]},
        "decode_stages": decode_stages,
        "roofline": roofline,
        "stages": stages,
        "topk_plus_attn": topk_plus_attn,
        "prefill_configs": prefill_configs or None,
        "measured_peaks": peaks,
        "train_align": train,
        "cpu_baseline": cpu,
        "cpu_baseline_single_thread": cpu1,
        "cpu_baseline_configs": cpu_cfgs,
        "cpu_model": cpu_model(),
        "cpu_threads": _blas_threads(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
