"""Write the oracle regression fixture (calls only the oracle and the input generators).

Run from the repository root:  python tests/golden/make_golden.py
The fixture records, for each small named workload, the sha256 of the seeded
inputs and of the oracle's quantized weights and scales, plus a few fp64
reference outputs.  A later change to the oracle's arithmetic that moves any of
these must say, in its commit message, which passage of the pages justifies it.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")


def main():
    rec = {}
    for name in ["tiny", "decode_gate_up", "decode_down"]:
        X, W = workloads.make(name)
        qw, sc = oracle.quantize(W)
        rows = [0] * 4
        cols = [0, 1, W.shape[0] // 2, W.shape[0] - 1]
        y, t = oracle.gemm_entries(X, qw, sc, rows, cols)
        rec[name] = {
            "sha256_X": workloads.sha256(X),
            "sha256_W": workloads.sha256(W),
            "sha256_qweight": workloads.sha256(qw),
            "sha256_scales": workloads.sha256(sc),
            "cols": cols,
            "y_ref": [float(v).hex() for v in y],
            "t_ref": [float(v).hex() for v in t],
        }
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
