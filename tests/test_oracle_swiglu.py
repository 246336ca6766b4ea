"""Pins of the oracle's fused gate/up SwiGLU (silu(X.gate) * (X.up)).

silu is checked against scipy's logistic function and its reflection
identity; the gate-then-up row order and the epilogue against a one-hot case
whose two dot products are exact and whose result is written out with
math.exp; the acceptance bound against perturbations just inside and
outside it.
"""

import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads


def test_silu_matches_logistic():
    v = np.concatenate([np.linspace(-30, 30, 601), [0.0, 1e-300, -1e-300, 700.0, -700.0, -1e5]])
    got = oracle.silu(v)
    want = v * expit(v)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([-1e5]))[0] == 0.0
    w = np.linspace(-20, 20, 81)
    assert np.allclose(oracle.silu(w) - oracle.silu(-w), w, rtol=0, atol=1e-13)


@pytest.mark.parametrize("qg,qu,s", [(7, 3, 0.5), (-8, 5, 0.25), (1, -7, 2.0), (0, 4, 1.0)])
def test_one_hot_gate_then_up(qg, qu, s):
    # x = e_0, gate row code qg, up row code qu at k = 0: g = qg*s, u = qu*s exactly
    K, F = 64, 3
    X = np.zeros((1, K), np.float32)
    X[0, 0] = 1.0
    nib = np.full((2 * F, K), 8, np.uint8)
    nib[1, 0] = qg + 8          # gate row 1
    nib[F + 1, 0] = qu + 8      # up row 1
    qw = oracle.pack(nib)
    sc = np.full((2 * F, K // 32), np.float32(s), np.float32)
    Y = oracle.swiglu(X, qw, sc)
    g, u = qg * s, qu * s
    assert Y.shape == (1, F)
    assert Y[0, 1] == pytest.approx(g / (1 + math.exp(-g)) * u, rel=1e-15, abs=0)
    assert Y[0, 0] == 0.0 and Y[0, 2] == 0.0


def test_bound_accepts_inside_and_rejects_outside():
    X, W = workloads.random_case(3, 2 * 40, 224, seed=9)
    qw, sc = oracle.quantize(W)
    ref = oracle.swiglu(X, qw, sc)
    b = oracle.swiglu_bound(X, qw, sc)
    assert np.all(b > 0)
    assert oracle.compare_swiglu(ref + 0.9 * b, X, qw, sc)["ok"]
    assert not oracle.compare_swiglu(ref + 1.1 * b, X, qw, sc)["ok"]
    # an fp32 evaluation from fp32 sums of g and u passes
    Y = oracle.gemm(X, qw, sc).astype(np.float32)
    g, u = Y[:, :40], Y[:, 40:]
    y32 = (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float32)
    assert oracle.compare_swiglu(y32, X, qw, sc)["ok"]
    # swapping gate and up is caught
    assert not oracle.compare_swiglu(oracle.silu(ref * 0 + oracle.gemm(X, qw, sc)[:, 40:]) *
                                     oracle.gemm(X, qw, sc)[:, :40], X, qw, sc)["ok"]
