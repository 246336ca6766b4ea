"""Pins of the oracle's grouped (MoE) GEMM and of the synthetic routing.

One expert reduces to the base product of the gathered rows; permuting the
slots of an expert permutes its output rows; a slot's row equals the base
product of its token and its expert on an exact integer case; malformed
routing is rejected; the routing generator gives every token topk distinct
experts and sorts slots by expert.
"""

import numpy as np
import pytest

import oracle
import workloads


def quantize_experts(W):
    qs = [oracle.quantize(W[e]) for e in range(W.shape[0])]
    return np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])


def test_routing_generator_is_well_formed():
    rng = np.random.default_rng(0)
    T, E, topk = 13, 9, 3
    ti, off = workloads.moe_routing(rng, T, E, topk)
    assert ti.dtype == np.int32 and off.dtype == np.int32
    assert ti.size == T * topk and off[0] == 0 and off[-1] == T * topk
    oracle.check_routing(ti, off, T, E)
    pairs = set()
    for e in range(E):
        toks = ti[off[e]:off[e + 1]]
        assert np.all(np.diff(toks) > 0)  # each token at most once per expert, ascending
        pairs |= {(int(t), e) for t in toks}
    assert all(sum(1 for (t, _) in pairs if t == tok) == topk for tok in range(T))


def test_single_expert_reduces_to_gemm_of_gathered_rows():
    X, W, _, _ = workloads.moe_case(6, 1, 1, 40, 96, seed=1)
    q, s = quantize_experts(W)
    ti = np.array([3, 0, 5, 5, 1], dtype=np.int32)
    off = np.array([0, 5], dtype=np.int32)
    Y = oracle.grouped_gemm(X, ti, off, q, s)
    assert np.array_equal(Y, oracle.gemm(X[ti], q[0], s[0]))


def test_slot_permutation_and_empty_experts():
    X, W, ti, off = workloads.moe_case(7, 5, 2, 30, 64, seed=2)
    q, s = quantize_experts(W)
    Y = oracle.grouped_gemm(X, ti, off, q, s)
    # permute the slots of every expert: rows follow
    perm = np.arange(ti.size)
    for e in range(5):
        perm[off[e]:off[e + 1]] = perm[off[e]:off[e + 1]][::-1]
    Yp = oracle.grouped_gemm(X, ti[perm], off, q, s)
    # the fp64 product's blocking may follow row position: equal to 1e-12
    assert np.allclose(Yp, Y[perm], rtol=1e-12, atol=1e-300)
    assert not np.allclose(Yp, Y, rtol=1e-6)
    # an expert with no slots changes nothing
    q2 = np.concatenate([q, q[:1]])
    s2 = np.concatenate([s, s[:1] * np.float32(3)])
    off2 = np.concatenate([off, off[-1:]])
    assert np.array_equal(oracle.grouped_gemm(X, ti, off2, q2, s2), Y)


def test_slot_equals_token_times_expert_exactly():
    # integer activations and codes with a power-of-two scale: every sum exact
    rng = np.random.default_rng(4)
    T, E, N, K = 4, 3, 8, 64
    X = rng.integers(-8, 9, (T, K)).astype(np.float32)
    nib = rng.integers(0, 16, (E, N, K)).astype(np.uint8)
    q = np.stack([oracle.pack(nib[e]) for e in range(E)])
    s = np.full((E, N, K // 32), np.float32(0.5), np.float32)
    ti = np.array([2, 0, 3, 1, 1], dtype=np.int32)
    off = np.array([0, 2, 2, 5], dtype=np.int32)   # expert 1 is empty
    Y = oracle.grouped_gemm(X, ti, off, q, s)
    owner = [0, 0, 2, 2, 2]
    for r in range(5):
        w = (nib[owner[r]].astype(np.int64) - 8) * 0.5
        assert np.array_equal(Y[r], X[ti[r]].astype(np.float64) @ w.T)


@pytest.mark.parametrize("ti,off", [([0, 1], [0, 1]), ([0, 1], [0, 2, 1]), ([0, 9], [0, 1, 2]),
                                    ([0, 1], [1, 1, 2]), ([-1, 0], [0, 1, 2])])
def test_malformed_routing_rejected(ti, off):
    X = np.zeros((3, 32), np.float32)
    q = np.zeros((2, 4, 4), np.int32)
    s = np.zeros((2, 4, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.grouped_gemm(X, np.array(ti, np.int32), np.array(off, np.int32), q, s)
