"""The oracle still reproduces the fixture written by tests/golden/make_golden.py."""
import json
import os

import pytest

import oracle
import workloads

FIX = os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")


@pytest.mark.parametrize("name", ["tiny", "decode_gate_up", "decode_down"])
def test_oracle_regression(name):
    rec = json.load(open(FIX))[name]
    X, W = workloads.make(name)
    assert workloads.sha256(X) == rec["sha256_X"]
    assert workloads.sha256(W) == rec["sha256_W"]
    qw, sc = oracle.quantize(W)
    assert workloads.sha256(qw) == rec["sha256_qweight"]
    assert workloads.sha256(sc) == rec["sha256_scales"]
    y, t = oracle.gemm_entries(X, qw, sc, [0] * len(rec["cols"]), rec["cols"])
    # fp64 dot products: allow a few ulps for a BLAS that sums in another order
    for got, want in zip(list(y) + list(t), rec["y_ref"] + rec["t_ref"]):
        assert got == pytest.approx(float.fromhex(want), rel=1e-12, abs=0)
