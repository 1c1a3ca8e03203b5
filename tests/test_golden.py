"""The oracle reproduces its frozen outputs (tests/golden/make_golden.py) for
the two small workloads, to 1e-12."""
import json
import os

import numpy as np

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "oracle_small_configs.json")


def test_oracle_matches_frozen_outputs():
    with open(GOLD) as f:
        g = json.load(f)
    for cid, rec in g["configs"].items():
        w = W.get(int(cid))
        assert rec["seed"] == w.seed and rec["scale"] == w.scale
        q, k, v, idx = W.make_inputs(w)
        O, L = oracle.attention(q, k, v, w.scale, kv_idx=idx, rows=np.array(rec["rows"]))
        np.testing.assert_allclose(O, np.array(rec["out"]), atol=1e-12, rtol=0)
        np.testing.assert_allclose(L, np.array(rec["lse"]), atol=1e-12, rtol=0)
