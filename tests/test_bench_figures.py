"""bench.py's algorithmic byte and flop counts and its rate arithmetic, checked
on the CPU against closed forms for the 128K chunked prefill (131072 causal
positions, k = 2048, 128 heads of 576 = 512 latent + 64 rope, indexer 64 x 128).
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from sparse_attention_18_amd import workloads as wk  # noqa: E402

WL = wk.CHUNKED_PREFILL_128K
POS = np.arange(WL.seq_len, dtype=np.int64)
L, K = 131072, 2048


def test_workload_shape():
    assert (WL.seq_len, WL.topk, WL.heads, WL.d_qk, WL.d_latent) == (L, K, 128, 576, 512)
    assert (WL.idx_heads, WL.idx_dim) == (64, 128)


def test_topk_bytes_closed_form():
    # every causal score read once (L (L + 1) / 2 of them) and k indices written per row
    want = 4.0 * L * (L + 1) / 2 + 4.0 * K * L
    assert bench.topk_bytes(WL, POS) == pytest.approx(want, rel=1e-12)
    assert want == pytest.approx(35.43e9, rel=1e-3)


def test_attention_bytes_and_flops_closed_form():
    # rows 0..k-1 select all p + 1 causal keys, the rest k
    pairs = K * (K + 1) / 2 + (L - K) * K
    per_pair = 576 * 2 + 4
    per_tok = 128 * 576 * 2 + 128 * 512 * 2
    want = pairs * per_pair + per_tok * L
    assert bench.attn_bytes(WL, POS) == pytest.approx(want, rel=1e-12)
    assert want / 32 == pytest.approx(10.762e9, rel=1e-3)          # per 4096-row chunk
    assert bench.attn_flops(WL, POS) == pytest.approx(pairs * 2 * 128 * (576 + 512), rel=1e-12)


def test_indexer_flops_closed_form():
    want = 2.0 * 64 * 128 * L * (L + 1) / 2
    assert bench.indexer_flops(WL, POS) == pytest.approx(want, rel=1e-12)


def test_stage_entry_rates():
    # 4 GB in 1 ms over two launches: 4 TB/s, half of the 8 TB/s peak
    e = bench.stage_entry(1.0, 2, "hbm", 4e9)
    assert e["achieved"] == pytest.approx(4000.0) and e["unit"] == "GB/s"
    assert e["frac"] == pytest.approx(0.5) and e["avg_launch_us"] == pytest.approx(500.0)
    # 2.5 PFLOP in 1 s against the 5.0 PFLOP/s FP8 peak
    e = bench.stage_entry(1000.0, 1, "mfma", 2.5e15)
    assert e["achieved"] == pytest.approx(2500.0) and e["frac"] == pytest.approx(0.5)
    # measured peaks give frac_measured against the faster of copy and read
    e = bench.stage_entry(1.0, 1, "hbm", 4e9, peaks={"hbm_copy_GBps": 5000.0, "hbm_read_GBps": 4000.0})
    assert e["frac_measured"] == pytest.approx(0.8)
