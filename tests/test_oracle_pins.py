"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against something fixed independently of it:
hand-decoded words, hand-quantized groups, closed forms, exact rational
arithmetic on tiny inputs, or invariants of the mathematics.  The format
facts pinned here are those of "The Quiet Commit: How a Single Documentation
Edit Marks the Completion of a Major Engineering Milestone", section "The
INT4 Milestone" (8 nibbles per int32 along the input dimension, value =
nibble - 8, fp32 group scales) and "The Silence of Success: A Single Line That
Speaks Volumes", section "What the Edit Actually Built" (groups of 32 input
columns, two 4-bit values per byte, dequantize-then-multiply).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def u32(v):
    return np.uint32(v).view(np.int32)


# ---------------------------------------------------------------- pack / unpack

def test_unpack_hand_decoded_words():
    # Low nibble first: 0x76543210 holds k = 0..7 as the values 0..7.
    q = np.array([[u32(0x76543210), u32(0xFEDCBA98)]], dtype=np.int32)
    nib = oracle.unpack(q)
    assert nib.tolist() == [[0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15]]
    # Two 4-bit values per byte: byte b of the little-endian word holds k=2b (low
    # half) and k=2b+1 (high half).
    b = q.view(np.uint8)[0, :4]
    assert [(int(x) & 15, int(x) >> 4) for x in b] == [(0, 1), (2, 3), (4, 5), (6, 7)]


def test_pack_each_value_at_each_position():
    for v in range(16):
        for i in range(8):
            nib = np.full((1, 8), 0, dtype=np.uint8)
            nib[0, i] = v
            w = oracle.pack(nib)
            assert int(w.view(np.uint32)[0, 0]) == v << (4 * i)
            assert oracle.unpack(w).tolist() == nib.tolist()


def test_pack_unpack_roundtrip_random():
    words = workloads.random_words((37, 24), seed=11)
    assert (words < 0).any()
    assert np.array_equal(oracle.pack(oracle.unpack(words)), words)
    rng = np.random.default_rng(5)
    nib = rng.integers(0, 16, size=(9, 64)).astype(np.uint8)
    assert np.array_equal(oracle.unpack(oracle.pack(nib)), nib)


# ---------------------------------------------------------------- dequantize

def test_dequant_hand_values():
    q = np.array([[u32(0x76543210), u32(0xFEDCBA98), u32(0x88888888), u32(0x00000000)]],
                 dtype=np.int32)
    s = np.array([[0.5]], dtype=np.float32)
    wd = oracle.dequantize(q, s)
    expect = [v * 0.5 for v in range(-8, 8)] + [0.0] * 8 + [-4.0] * 8
    assert wd.dtype == np.float32
    assert wd[0].tolist() == expect


def test_dequant_is_one_rounded_product():
    # fl32((q-8)*s) equals the exact product rounded once to fp32: the fp64
    # product of a 4-bit integer and an fp32 value is exact.
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=(64, 8), dtype=np.uint64).astype(np.uint32)
    s = bits.view(np.float32)
    s = np.where(np.isfinite(s), s, np.float32(1.5)).astype(np.float32)
    nib = rng.integers(0, 16, size=(64, 256)).astype(np.uint8)
    with np.errstate(over="ignore"):
        wd = oracle.dequantize(oracle.pack(nib), s)
        exact = (nib.astype(np.float64) - 8.0) * np.repeat(s.astype(np.float64), 32, axis=1)
        assert np.array_equal(wd, exact.astype(np.float32))


def test_dequant_rejects_bad_scale_shape():
    with pytest.raises(ValueError):
        oracle.dequantize(np.zeros((2, 8), np.int32), np.zeros((2, 3), np.float32))


# ---------------------------------------------------------------- quantize

def _hand_group():
    # max|w| = 7 so scale = 1 exactly; the remaining values exercise ties to even.
    w = [7.0, -7.0, 3.5, 2.5, -2.5, 0.5, 1.5, -0.5,
         6.6, -3.2, 0.0, 1.0, -6.5, 4.5, 5.49, -1.51] + [0.0] * 16
    # rint: 4 (3.5), 2 (2.5), -2 (-2.5), 0 (0.5), 2 (1.5), -0 (-0.5), 7 (6.6),
    # -3 (-3.2), 0, 1, -6 (-6.5), 4 (4.5), 5 (5.49), -2 (-1.51)
    q = [7, -7, 4, 2, -2, 0, 2, 0, 7, -3, 0, 1, -6, 4, 5, -2] + [0] * 16
    return np.array(w, np.float32), [v + 8 for v in q]


def test_quantize_hand_group():
    w, nib = _hand_group()
    qw, sc = oracle.quantize(w[None, :])
    assert sc.tolist() == [[1.0]]
    assert oracle.unpack(qw)[0].tolist() == nib
    # nibbles 0..7 are 15,1,12,10,6,8,10,8 -> 0x8A86AC1F, written high digit first
    assert int(qw.view(np.uint32)[0, 0]) == 0x8A86AC1F


def test_quantize_hand_group_second_word():
    w, nib = _hand_group()
    qw, _ = oracle.quantize(w[None, :])
    # nibbles 8..15 are 15,5,8,9,2,12,13,6 -> 0x6DC2985F
    assert int(qw.view(np.uint32)[0, 1]) == 0x6DC2985F
    assert int(qw.view(np.uint32)[0, 2]) == 0x88888888
    assert int(qw.view(np.uint32)[0, 3]) == 0x88888888


def test_quantize_scale_quarter():
    # max|w| = 1.75 -> scale = 1.75/7 = 0.25 exactly; w/0.25 is exact.
    w = np.zeros((1, 32), np.float32)
    w[0, :6] = [1.75, -0.25, 0.375, 0.625, -1.75, 0.125]
    qw, sc = oracle.quantize(w)
    assert sc.tolist() == [[0.25]]
    # 7, -1, 1.5->2, 2.5->2, -7, 0.5->0
    assert oracle.unpack(qw)[0, :6].tolist() == [15, 7, 10, 10, 1, 8]


def test_quantize_zero_and_underflow_groups():
    w = np.zeros((2, 64), np.float32)
    w[1, 32] = np.float32(2.0 ** -149)   # smallest subnormal: max/7 underflows to 0
    w[1, 33] = np.float32(-1e-46)        # rounds to -0 or tiny, still < max
    qw, sc = oracle.quantize(w)
    assert sc.tolist() == [[0.0, 0.0], [0.0, 0.0]]
    assert np.all(oracle.unpack(qw) == 8)


def test_quantize_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 48), np.float32))
    w = np.zeros((2, 64), np.float32)
    w[1, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize(w)
    w[1, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize(w)


def test_quantize_roundtrip_power_of_two_scales():
    # With scales 2^e and a +-7 in every group, dequant then quantize returns
    # the same codes and scales bit for bit.
    rng = np.random.default_rng(7)
    N, K = 16, 256
    G = K // 32
    centred = rng.integers(-7, 8, size=(N, G, 32))
    centred[:, :, 0] = np.where(rng.random((N, G)) < 0.5, 7, -7)
    nib = (centred + 8).reshape(N, K).astype(np.uint8)
    sc = np.ldexp(np.float32(1.0), rng.integers(-20, 10, size=(N, G))).astype(np.float32)
    qw = oracle.pack(nib)
    qw2, sc2 = oracle.quantize(oracle.dequantize(qw, sc))
    assert np.array_equal(sc2, sc)
    assert np.array_equal(qw2, qw)


def test_quantize_error_bound_and_extremes():
    # Rounding to nearest: |w - dequant| <= scale/2 (plus fp32 slack), and the
    # largest |w| of every non-zero group lands on +-7.
    x, W = workloads.random_case(1, 96, 512, seed=9, w_kind="outlier")
    qw, sc = oracle.quantize(W)
    wd = oracle.dequantize(qw, sc)
    s = np.repeat(sc, 32, axis=1).astype(np.float64)
    err = np.abs(W.astype(np.float64) - wd.astype(np.float64))
    assert np.all(err <= 0.5 * s * (1 + 4e-6) + 1e-30)
    nib = oracle.unpack(qw).reshape(96, 16, 32).astype(int)
    assert np.all(np.max(np.abs(nib - 8), axis=2) == 7)
    assert not np.any(nib == 0)                      # -8 is never produced here


def test_quantize_symmetry_and_scaling():
    _, W = workloads.random_case(1, 40, 256, seed=13)
    qa, sa = oracle.quantize(W)
    qb, sb = oracle.quantize(-W)
    assert np.array_equal(sa, sb)
    assert np.array_equal(16 - oracle.unpack(qa).astype(int), oracle.unpack(qb).astype(int))
    qc, sc = oracle.quantize((W * np.float32(8.0)).astype(np.float32))
    assert np.array_equal(qc, qa)
    assert np.array_equal(sc, sa * np.float32(8.0))


# ---------------------------------------------------------------- the product

def _exact(X, qweight, scales):
    """Exact rational product from raw words, in pure Python integers."""
    M, K = X.shape
    N = qweight.shape[0]
    Y = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        w = []
        for k in range(K):
            word = int(qweight[n, k // 8]) & 0xFFFFFFFF
            nib = (word >> (4 * (k % 8))) & 0xF
            exact_w = (nib - 8) * Fraction(float(scales[n, k // 32]))
            # the dequantized weight is that product rounded once to fp32 (a
            # 4-bit integer times an fp32 value is exact as a Python float)
            w.append(Fraction(float(np.float32(float(exact_w)))))
        for m in range(M):
            Y[m][n] = sum((Fraction(float(X[m, k])) * w[k] for k in range(K)), Fraction(0))
    return Y


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 32, 0), (2, 3, 64, 1), (3, 5, 32, 2), (3, 2, 96, 3)])
def test_gemm_matches_exact_rationals(M, N, K, seed):
    X, W = workloads.random_case(M, N, K, seed)
    qw, sc = oracle.quantize(W)
    Y = oracle.gemm(X, qw, sc)
    T = oracle.abs_gemm(X, qw, sc)
    ex = _exact(X, qw, sc)
    assert Y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            assert abs(Y[m, n] - float(ex[m][n])) <= K * 2.0 ** -52 * T[m, n] + 1e-300


def test_gemm_integer_case_is_exact():
    X, nib = workloads.integer_case(3, 4, 96, seed=21)
    qw = oracle.pack(nib)
    sc = np.full((4, 3), np.float32(2.0 ** -3))
    Y = oracle.gemm(X, qw, sc)
    ex = _exact(X, qw, sc)
    assert Y.tolist() == [[float(v) for v in row] for row in ex]


def test_gemm_one_hot_word():
    # All nibbles 8 (weight 0) except nibble i of word j = 9 (weight +1*s):
    # Y[:, n] is s * X[:, 8j + i] exactly.
    rng = np.random.default_rng(1)
    X = rng.standard_normal((3, 64)).astype(np.float32)
    qw = np.full((2, 8), u32(0x88888888), dtype=np.int32)
    j, i = 5, 3
    qw[1, j] = u32(0x88888888 ^ (0x1 << (4 * i)))     # 8 -> 9 at nibble i
    sc = np.array([[0.75, 0.75], [0.75, 0.75]], np.float32)
    Y = oracle.gemm(X, qw, sc)
    assert np.all(Y[:, 0] == 0.0)
    assert np.array_equal(Y[:, 1], X[:, 8 * j + i].astype(np.float64) * 0.75)


def test_gemm_invariants():
    X, W = workloads.random_case(4, 7, 128, seed=5)
    qw, sc = oracle.quantize(W)
    assert np.all(oracle.gemm(np.zeros_like(X), qw, sc) == 0.0)
    Y = oracle.gemm(X, qw, sc)
    T = oracle.abs_gemm(X, qw, sc)
    assert np.array_equal(oracle.gemm((X * np.float32(4.0)).astype(np.float32), qw, sc), 4.0 * Y)
    perm = np.array([2, 0, 3, 1])
    assert np.allclose(oracle.gemm(X[perm], qw, sc), Y[perm], rtol=0, atol=1e-12)
    X2, _ = workloads.random_case(4, 7, 128, seed=6)
    a, b = np.float32(0.5), np.float32(-2.0)
    lin = oracle.gemm((a * X + b * X2).astype(np.float32), qw, sc)
    ref = 0.5 * Y - 2.0 * oracle.gemm(X2, qw, sc)
    T2 = 0.5 * T + 2.0 * oracle.abs_gemm(X2, qw, sc)
    assert np.all(np.abs(lin - ref) <= oracle.bound(T2))
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros((1, 48), np.float32), np.zeros((1, 6), np.int32),
                    np.zeros((1, 1), np.float32))


def test_gemm_entries_agree_with_full_product():
    X, W = workloads.random_case(5, 9, 160, seed=8)
    qw, sc = oracle.quantize(W)
    Y = oracle.gemm(X, qw, sc)
    T = oracle.abs_gemm(X, qw, sc)
    rows, cols = [0, 4, 2, 3], [8, 0, 5, 5]
    y, t = oracle.gemm_entries(X, qw, sc, rows, cols)
    assert np.allclose(y, Y[rows, cols], rtol=1e-14, atol=0)
    assert np.allclose(t, T[rows, cols], rtol=1e-14, atol=0)


# ---------------------------------------------------------------- acceptance

def test_bound_literals():
    assert oracle.bound(0.0) == pytest.approx(1e-6, rel=1e-15)
    assert oracle.bound(1.0) == pytest.approx(1.1e-5, rel=1e-15)


def test_compare_accepts_inside_and_rejects_outside():
    X, W = workloads.random_case(2, 6, 64, seed=4)
    qw, sc = oracle.quantize(W)
    Y = oracle.gemm(X, qw, sc)
    T = oracle.abs_gemm(X, qw, sc)
    assert oracle.compare(Y, X, qw, sc)["ok"]
    assert oracle.compare(Y + 0.9 * oracle.bound(T), X, qw, sc)["ok"]
    assert not oracle.compare(Y + 1.1 * oracle.bound(T), X, qw, sc)["ok"]
    bad = Y.copy()
    bad[1, 2] = np.nan
    assert not oracle.compare(bad, X, qw, sc)["ok"]


@pytest.mark.parametrize("name", ["tiny", "decode_down"])
def test_negative_control_unquantized_weights_miss(name):
    # Quantization must really change the result: X . W^T with the unquantized
    # weights lies outside the tolerance of the quantized product.
    X, W = workloads.make(name)
    qw, sc = oracle.quantize(W)
    plain = X.astype(np.float64) @ W.astype(np.float64).T
    assert not oracle.compare(plain, X, qw, sc)["ok"]
