"""Pins of the oracle's grouped repack (pack_grouped / unpack_grouped) against
the layout stated for w4a16_grouped_pack, with index arithmetic written out
here from that statement (not taken from the oracle)."""

import numpy as np
import pytest

import oracle
import workloads


def words_and_scales(E, N, K, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-2**31, 2**31, size=(E, N, K // 8), dtype=np.int64).astype(np.int32)
    s = rng.uniform(0.001, 1.0, size=(E, N, K // 32)).astype(np.float32)
    return q, s


def geometry(E, N, K):
    G = K // 32
    T16, S4 = -(-N // 16), -(-G // 4)
    return G, T16, S4, E * T16 * S4


@pytest.mark.parametrize("E,N,K", [(1, 16, 128), (2, 20, 160), (3, 7, 96), (1, 33, 416)])
def test_round_trip(E, N, K):
    q, s = words_and_scales(E, N, K, E + N + K)
    p = oracle.pack_grouped(q, s)
    assert p.size == geometry(E, N, K)[3] * 1280
    q2, s2 = oracle.unpack_grouped(p, E, N, K)
    assert np.array_equal(q2, q) and np.array_equal(s2.view(np.uint32), s.view(np.uint32))


def test_every_word_and_scale_at_its_stated_offset():
    E, N, K = 2, 19, 224
    q, s = words_and_scales(E, N, K, 7)
    G, T16, S4, B = geometry(E, N, K)
    p = oracle.pack_grouped(q, s)
    w32 = p[:B * 1024].view(np.uint32)
    f32 = p[B * 1024:].view(np.float32)
    qu = q.view(np.uint32)
    for e in range(E):
        for n in range(N):
            t, c = n // 16, n % 16
            for g in range(G):
                st, qq = g // 4, g % 4
                b = (e * T16 + t) * S4 + st
                for R in range(4):
                    chunk = b * 64 + c + 16 * R        # 16-byte chunk index
                    assert w32[chunk * 4 + qq] == qu[e, n, 4 * g + R]
                assert f32[(b * 16 + c) * 4 + qq] == s[e, n, g]


def test_padding_is_code_zero_and_scale_zero():
    E, N, K = 1, 18, 160            # rows 18..31 and groups 5..7 are padding
    q, s = words_and_scales(E, N, K, 3)
    G, T16, S4, B = geometry(E, N, K)
    p = oracle.pack_grouped(q, s)
    w32 = p[:B * 1024].view(np.uint32).reshape(B, 64, 4)
    f32 = p[B * 1024:].view(np.float32).reshape(B, 16, 4)
    for t in range(T16):
        for st in range(S4):
            b = t * S4 + st
            for c in range(16):
                for qq in range(4):
                    pad = 16 * t + c >= N or 4 * st + qq >= G
                    if pad:
                        assert f32[b, c, qq] == 0.0
                        for R in range(4):
                            assert w32[b, c + 16 * R, qq] == 0x88888888


def test_grouped_gemm_through_packed_bytes():
    """Each weight fetched through the packed bytes (plain loops) gives the
    oracle's grouped product; a wrong lane order does not."""
    T, E, topk, N, K = 5, 3, 2, 18, 160
    X, W, ti, off = workloads.moe_case(T, E, topk, N, K, seed=11)
    qs = [oracle.quantize(W[e]) for e in range(E)]
    q = np.stack([a for a, _ in qs])
    s = np.stack([b for _, b in qs])
    G, T16, S4, B = geometry(E, N, K)
    p = oracle.pack_grouped(q, s)
    w32 = p[:B * 1024].view(np.uint32)
    f32 = p[B * 1024:].view(np.float32)

    def dequant(e, swap_lanes=False):
        Wd = np.zeros((N, K))
        for n in range(N):
            t, c = n // 16, n % 16
            for g in range(G):
                st, qq = g // 4, g % 4
                b = (e * T16 + t) * S4 + st
                sc = np.float64(f32[(b * 16 + c) * 4 + qq])
                for R in range(4):
                    lane = (R + 16 * c) % 64 if swap_lanes else c + 16 * R
                    word = int(w32[(b * 64 + lane) * 4 + qq])
                    for i in range(8):
                        nib = (word >> (4 * i)) & 0xF
                        Wd[n, 32 * g + 8 * R + i] = float(np.float32((nib - 8) * sc))
        return Wd

    ref = oracle.grouped_gemm(X, ti, off, q, s)
    Y = np.zeros_like(ref)
    Yw = np.zeros_like(ref)
    for e in range(E):
        Wd, Ww = dequant(e), dequant(e, swap_lanes=True)
        for r in range(off[e], off[e + 1]):
            Y[r] = X[ti[r]].astype(np.float64) @ Wd.T
            Yw[r] = X[ti[r]].astype(np.float64) @ Ww.T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)
    assert not np.allclose(Yw, ref, rtol=1e-3)
