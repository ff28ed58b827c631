"""The oracle still reproduces its committed regression fixture.

tests/golden/tiny_dsa.json was written by tests/golden/make_golden.py, which
calls only the oracle; this guards the oracle against silent drift.  It is a
regression pin, not an independent one (those live in the other
test_oracle_* files).
"""
import json
import os

import numpy as np

from oracle import dequantize, forward_rows

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_committed_fixture():
    with open(os.path.join(HERE, "golden", "tiny_dsa.json")) as f:
        doc = json.load(f)
    inp = {k: (np.array(v) if isinstance(v, list) else v) for k, v in doc["inputs"].items()}
    qd = dequantize(inp["q_fp8"].astype(np.uint8), inp["q_scale"].astype(np.float32))
    kd = dequantize(inp["k_fp8"].astype(np.uint8), inp["k_scale"].astype(np.float32))
    L = qd.shape[0]
    scores, idx, out, lse = forward_rows(qd, inp["w"].astype(np.float32).astype(np.float64), kd,
                                         np.arange(L), inp["q"], inp["kv"], inp["topk"],
                                         inp["scale"], inp["d_latent"])
    for a, b in zip(scores, doc["scores"]):
        np.testing.assert_allclose(a, b, rtol=1e-15, atol=0)
    np.testing.assert_array_equal(idx, doc["idx"])
    np.testing.assert_allclose(out, doc["out"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, doc["lse"], rtol=1e-14, atol=1e-15)
    # the pattern has exact ties in the indexer scores, so the tie rule is exercised
    assert any(len(set(s)) < len(s) for s in doc["scores"])
