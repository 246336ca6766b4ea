"""Pins of the oracle's split-path packed layout (pack_split / unpack_split).

The layout is the library's own (the pages describe no repack; the library
adds a one-time repack into layouts private to its kernels); it moves bits
only.  Pinned by: a round trip that
restores every input bit, the padding contents and size, and a GEMM computed
by plain loops that fetch each weight and scale through the packed bytes,
which must equal the oracle's product of the unpacked operands exactly.
"""

import numpy as np
import pytest

import oracle
import workloads


@pytest.mark.parametrize("N,K", [(1, 32), (2, 96), (64, 64), (65, 224), (130, 320), (7, 7168)])
def test_pack_round_trip_restores_every_bit(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    q = rng.integers(0, 2**32, (N, K // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    s = rng.standard_normal((N, K // 32)).astype(np.float32)
    p = oracle.pack_split(q, s)
    S, T = -(-N // 64), -(-(K // 32) // 2)
    assert p.dtype == np.uint8 and p.size == S * T * 2560
    q2, s2 = oracle.unpack_split(p, N, K)
    assert np.array_equal(q2, q) and np.array_equal(s2.view(np.uint32), s.view(np.uint32))


def test_pack_padding_is_code_zero_and_scale_zero():
    # N = 2 rows, K = 96 (3 groups: the second group of stage 1 is padding)
    N, K = 2, 96
    q = np.arange(N * K // 8, dtype=np.int32).reshape(N, K // 8) + 1
    s = np.array([[1.5, 2.5, 3.5], [4.5, 5.5, 6.5]], dtype=np.float32)
    p = oracle.pack_split(q, s)
    words = p[:2 * 2 * 64 * 16].view(np.uint32).reshape(2, 2, 64, 4)  # [stage][g][row][word]
    sc = p[2 * 2 * 64 * 16:].view(np.float32).reshape(2, 64, 2)      # [stage][row][g]
    # stage 1, group 1 is past G = 3: every row holds code 0 and scale 0
    assert np.all(words[1, 1] == 0x88888888) and np.all(sc[1, :, 1] == 0.0)
    # rows 2..63 are past N
    assert np.all(words[:, :, 2:] == 0x88888888) and np.all(sc[:, 2:] == 0.0)
    # a real entry: row 1, group 2 (stage 1, g 0) holds that group's 4 words
    assert np.array_equal(words[1, 0, 1].view(np.int32), q[1, 8:12]) and sc[1, 1, 0] == 6.5
    # the padding decodes to weight 0
    assert np.all(oracle.unpack(np.full((1, 1), 0x88888888, np.uint32).view(np.int32)) == 8)


def test_gemm_through_packed_bytes_equals_oracle():
    # fetch every weight nibble and scale through the packed layout with plain
    # loops, multiply-accumulate in fp64, compare with the oracle's product
    M, N, K = 2, 67, 160
    X, W = workloads.random_case(M, N, K, seed=5)
    q, s = oracle.quantize(W)
    p = oracle.pack_split(q, s)
    G, T = K // 32, -(-(K // 32) // 2)
    S = -(-N // 64)
    words = p[:S * T * 2048].view(np.uint32)
    sc = p[S * T * 2048:].view(np.float32)
    Y = np.zeros((M, N))
    for n in range(N):
        slab, r = divmod(n, 64)
        for k in range(K):
            gg, kk = divmod(k, 32)
            t, g = divmod(gg, 2)
            word = words[(((slab * T + t) * 2 + g) * 64 + r) * 4 + kk // 8]
            nib = (int(word) >> (4 * (kk % 8))) & 15
            w = np.float32(np.float32(nib - 8) * sc[(slab * T + t) * 128 + 2 * r + g])
            Y[:, n] += X[:, k].astype(np.float64) * float(w)
    # same exact fp64 products; only the summation order differs
    ref = oracle.gemm(X, q, s)
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-300)
    assert not np.allclose(Y[:, :3], oracle.gemm(X, q, s * np.float32(1.001))[:, :3], rtol=1e-6)
