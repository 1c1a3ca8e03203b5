"""Writes oracle_small_configs.json: float64 oracle outputs for the two small
workloads (one-head decode, hd 64, s_k 128; one-head prefill, hd 128, s_k 256),
on their seeded inputs.  Calls only ``oracle`` and ``workloads``.

The file freezes the oracle: a later change to its arithmetic shows up as a
failing ``tests/test_golden.py`` and must be justified by the passage it
follows.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as W  # noqa: E402

ROWS = {1: [0], 2: [0, 1, 63, 64, 127]}


def main():
    out = {"recipe": "workloads.make_inputs(workloads.get(cid)); oracle.attention "
                     "(float64) on the listed flat rows",
           "configs": {}}
    for cid, rows in ROWS.items():
        w = W.get(cid)
        q, k, v, idx = W.make_inputs(w)
        O, L = oracle.attention(q, k, v, w.scale, kv_idx=idx, rows=np.array(rows))
        out["configs"][str(cid)] = {
            "workload": w.describe(), "seed": w.seed, "scale": w.scale,
            "rows": rows, "out": O.tolist(), "lse": L.tolist()}
    with open(os.path.join(HERE, "oracle_small_configs.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
