"""Writes tests/golden/tiny_dsa.json from the float64 oracle alone.

The inputs are fixed integer patterns (no random draws), small enough to read:
FP8 codes and scales for a 12-token sequence with 2 indexer heads of width 4,
top-k = 3, and a 2-head attention over 3 latent + 2 rope columns.  Run from
the repository root: ``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import dequantize, forward_rows  # noqa: E402


def fixed_inputs():
    L, HI, dI, H, dl, dr = 12, 2, 4, 2, 3, 2
    r = np.arange(L)[:, None, None]
    j = np.arange(HI)[None, :, None]
    d = np.arange(dI)[None, None, :]
    # codes cycle through e4m3fn values 0.5, 1, 1.5, 2, -1, -0.5 (0x30 0x38 0x3C 0x40 0xB8 0xB0)
    table = np.array([0x30, 0x38, 0x3C, 0x40, 0xB8, 0xB0], dtype=np.uint8)
    q_fp8 = table[(3 * r + 5 * j + 7 * d) % 6]
    k_fp8 = table[(2 * np.arange(L)[:, None] + 3 * np.arange(dI)[None, :]) % 6]
    q_scale = (1.0 + (np.arange(L) % 3) / 4.0).astype(np.float32)
    k_scale = (0.5 + (np.arange(L) % 4) / 8.0).astype(np.float32)
    w = ((np.arange(L)[:, None] + 2 * np.arange(HI)[None, :]) % 5 / 4.0).astype(np.float32)
    D = dl + dr
    q = ((np.arange(L)[:, None, None] * 3 + np.arange(H)[None, :, None] * 5
          + np.arange(D)[None, None, :] * 7) % 9 - 4) / 4.0
    kv = ((np.arange(L)[:, None] * 5 + np.arange(D)[None, :] * 3) % 7 - 3) / 2.0
    return dict(q_fp8=q_fp8, k_fp8=k_fp8, q_scale=q_scale, k_scale=k_scale, w=w, q=q, kv=kv,
                topk=3, scale=0.5, d_latent=dl)


def main():
    inp = fixed_inputs()
    qd = dequantize(inp["q_fp8"], inp["q_scale"])
    kd = dequantize(inp["k_fp8"], inp["k_scale"])
    L = qd.shape[0]
    scores, idx, out, lse = forward_rows(qd, inp["w"].astype(np.float64), kd, np.arange(L),
                                         inp["q"], inp["kv"], inp["topk"], inp["scale"],
                                         inp["d_latent"])
    doc = {
        "what": "oracle regression fixture: fixed integer-pattern inputs, float64 oracle outputs",
        "writer": "tests/golden/make_golden.py (calls only oracle/)",
        "inputs": {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in inp.items()},
        "scores": [s.tolist() for s in scores],
        "idx": idx.tolist(),
        "out": out.tolist(),
        "lse": lse.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_dsa.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
