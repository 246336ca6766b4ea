"""GPU parity of the grouped (MoE) W4A16 GEMM (w4a16_gemm_grouped) against the oracle."""

import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_only_03_amd import binding  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    binding.load()
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def quantize_experts(W):
    qs = [oracle.quantize(W[e]) for e in range(W.shape[0])]
    return np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])


def run(X, ti, off, q, s, dev, Y=None):
    out = binding.w4a16_gemm_grouped(to_dev(X, dev), to_dev(ti, dev), to_dev(off, dev),
                                     to_dev(q, dev), to_dev(s, dev), Y)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("T,E,topk,N,K", [
    (1, 1, 1, 33, 32),        # one slot, one expert
    (7, 5, 2, 70, 96),        # ragged everything
    (16, 32, 4, 64, 256),     # many experts, some empty
    (1, 64, 8, 40, 224),      # one token: most experts empty
    (32, 4, 2, 96, 512),      # ~16 slots per expert (4-row chunks)
    (9, 3, 2, 257, 2048),     # 2-row chunks
    (4, 8, 8, 128, 7168),     # every expert used, K of the gate+up width
    (3, 4, 2, 100, 288),      # 1.5 slots per expert: 2-row chunks on the matrix cores
    (6, 4, 2, 48, 16384 + 32),  # K too long for 4 staged rows: fewer rows per chunk
])
def test_grouped_shapes(dev, T, E, topk, N, K):
    say(f"grouped T={T} E={E} topk={topk} N={N} K={K}")
    X, W, ti, off = workloads.moe_case(T, E, topk, N, K, seed=T * 31 + E * 7 + N + K)
    q, s = quantize_experts(W)
    v = oracle.compare_grouped(run(X, ti, off, q, s, dev), X, ti, off, q, s)
    say(f"  empty experts {int(np.sum(np.diff(off) == 0))}, max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


def test_grouped_all_slots_on_one_expert(dev):
    T, E, N, K = 12, 6, 50, 160
    X, W, _, _ = workloads.moe_case(T, E, 1, N, K, seed=8)
    q, s = quantize_experts(W)
    ti = np.arange(T, dtype=np.int32)[::-1].copy()
    off = np.array([0, 0, 0, T, T, T, T], dtype=np.int32)
    v = oracle.compare_grouped(run(X, ti, off, q, s, dev), X, ti, off, q, s)
    assert v["ok"], v


def test_grouped_integer_exact(dev):
    rng = np.random.default_rng(4)
    T, E, N, K = 6, 4, 40, 512
    X = rng.integers(-8, 9, (T, K)).astype(np.float32)
    nib = rng.integers(0, 16, (E, N, K)).astype(np.uint8)
    q = np.stack([oracle.pack(nib[e]) for e in range(E)])
    s = np.full((E, N, K // 32), np.float32(0.25), np.float32)
    ti = np.array([0, 5, 1, 2, 3, 4, 0, 1, 2], dtype=np.int32)
    off = np.array([0, 2, 2, 6, 9], dtype=np.int32)
    Y = run(X, ti, off, q, s, dev)
    assert np.array_equal(Y.astype(np.float64), oracle.grouped_gemm(X, ti, off, q, s))


def test_grouped_guard_band_and_determinism(dev):
    T, E, topk, N, K = 5, 4, 2, 45, 96
    X, W, ti, off = workloads.moe_case(T, E, topk, N, K, seed=3)
    q, s = quantize_experts(W)
    R = ti.size
    pad = 4096
    buf = torch.full((pad + R * N + pad,), 0x7FC0DEAD, dtype=torch.int32, device=dev)
    Y = buf[pad:pad + R * N].view(torch.float32).view(R, N)
    a = run(X, ti, off, q, s, dev, Y)
    host = buf.cpu().numpy().view(np.uint32)
    assert np.all(host[:pad] == 0x7FC0DEAD) and np.all(host[pad + R * N:] == 0x7FC0DEAD)
    b = run(X, ti, off, q, s, dev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert oracle.compare_grouped(a, X, ti, off, q, s)["ok"]


def test_grouped_moe_decode_full_size(dev):
    """The moe_decode workload as timed (16 tokens, top-4 of 32 experts, N=1024,
    K=7168): every output of the public-layout and packed kernels against the
    oracle, and the two bit for bit (the same matrix-core kernel)."""
    X, W, ti, off = workloads.make_moe("moe_decode")
    T, E, N, K = X.shape[0], W.shape[0], W.shape[1], W.shape[2]
    say(f"grouped moe_decode full size T={T} E={E} N={N} K={K}, {int(np.sum(np.diff(off) == 0))} empty")
    q, s = quantize_experts(W)
    del W
    Yu = run(X, ti, off, q, s, dev)
    packed = binding.w4a16_grouped_pack(to_dev(q, dev), to_dev(s, dev))
    Yp = binding.w4a16_gemm_grouped_packed(to_dev(X, dev), to_dev(ti, dev), to_dev(off, dev),
                                           packed, E, N)
    torch.cuda.synchronize()
    Yp = Yp.cpu().numpy()
    assert np.array_equal(Yp.view(np.uint32), Yu.view(np.uint32))
    v = oracle.compare_grouped(Yu, X, ti, off, q, s)
    say(f"  max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


def test_grouped_many_experts_fallback(dev):
    # more experts than the matrix-core kernel's work list takes: the
    # LDS-staged FMA kernel runs instead
    T, E, topk, N, K = 6, 4100, 3, 20, 96
    say(f"grouped fallback E={E}")
    X, W, ti, off = workloads.moe_case(T, E, topk, N, K, seed=21)
    assert binding.w4a16_grouped_kernel(T, ti.size, E, N, K) == binding.W4A16_GROUPED_ROWS
    q, s = quantize_experts(W)
    v = oracle.compare_grouped(run(X, ti, off, q, s, dev), X, ti, off, q, s)
    assert v["ok"], v


def test_grouped_long_k_fallback(dev):
    # K too long to stage even one token row in LDS: the kernel that reads
    # activations from memory runs instead
    T, E, topk, N, K = 3, 2, 1, 8, 40960 + 32
    say(f"grouped fallback K={K}")
    X, W, ti, off = workloads.moe_case(T, E, topk, N, K, seed=22)
    assert binding.w4a16_grouped_kernel(T, ti.size, E, N, K) == binding.W4A16_GROUPED_GEMV
    q, s = quantize_experts(W)
    v = oracle.compare_grouped(run(X, ti, off, q, s, dev), X, ti, off, q, s)
    assert v["ok"], v


# ---------------------------------------------------------------- packed layout

def dev_words(E, N, K, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-2**31, 2**31, size=(E, N, K // 8), dtype=np.int64).astype(np.int32)
    s = rng.uniform(0.001, 1.0, size=(E, N, K // 32)).astype(np.float32)
    return q, s


@pytest.mark.parametrize("E,N,K", [(2, 20, 160), (3, 7, 96), (1, 33, 416), (4, 64, 7168)])
def test_grouped_pack_bit_exact(dev, E, N, K):
    say(f"grouped pack E={E} N={N} K={K}")
    q, s = dev_words(E, N, K, E * 7 + N + K)
    packed = binding.w4a16_grouped_pack(to_dev(q, dev), to_dev(s, dev))
    torch.cuda.synchronize()
    ref = oracle.pack_grouped(q, s)
    got = packed.cpu().numpy()[:ref.size]
    assert packed.numel() == ref.size == binding.w4a16_grouped_pack_bytes(E, N, K)
    assert np.array_equal(got, ref)


def test_grouped_pack_full_size_sampled(dev):
    """The moe_decode expert shape: sampled words and scales sit at the offsets
    the layout states (index arithmetic written out here)."""
    wl = workloads.MOE_WORKLOADS["moe_decode"]
    E, N, K = wl.E, wl.N, wl.K
    say(f"grouped pack full size E={E} N={N} K={K}")
    q, s = dev_words(E, N, K, 99)
    packed = binding.w4a16_grouped_pack(to_dev(q, dev), to_dev(s, dev))
    torch.cuda.synchronize()
    p = packed.cpu().numpy()
    G, T16, S4 = K // 32, -(-N // 16), -(-(K // 32) // 4)
    B = E * T16 * S4
    w32 = p[:B * 1024].view(np.uint32)
    f32 = p[B * 1024:B * 1280].view(np.float32)
    rng = np.random.default_rng(5)
    qu = q.view(np.uint32)
    for _ in range(4000):
        e, n, g, R = rng.integers(E), rng.integers(N), rng.integers(G), rng.integers(4)
        b = (e * T16 + n // 16) * S4 + g // 4
        assert w32[(b * 64 + n % 16 + 16 * R) * 4 + g % 4] == qu[e, n, 4 * g + R]
        assert f32[(b * 16 + n % 16) * 4 + g % 4] == s[e, n, g]


@pytest.mark.parametrize("T,E,topk,N,K", [
    (7, 5, 2, 70, 96),
    (16, 32, 4, 64, 256),
    (1, 64, 8, 40, 224),
    (32, 4, 2, 96, 512),
    (3, 4, 2, 100, 288),
    (4, 8, 8, 128, 7168),
])
def test_grouped_packed_matches_unpacked(dev, T, E, topk, N, K):
    say(f"grouped packed T={T} E={E} topk={topk} N={N} K={K}")
    X, W, ti, off = workloads.moe_case(T, E, topk, N, K, seed=T * 13 + E + N + K)
    assert binding.w4a16_grouped_kernel(T, ti.size, E, N, K) == binding.W4A16_GROUPED_MFMA
    q, s = quantize_experts(W)
    packed = binding.w4a16_grouped_pack(to_dev(q, dev), to_dev(s, dev))
    Yp = binding.w4a16_gemm_grouped_packed(to_dev(X, dev), to_dev(ti, dev), to_dev(off, dev),
                                           packed, E, N)
    torch.cuda.synchronize()
    Yp = Yp.cpu().numpy()
    Yu = run(X, ti, off, q, s, dev)
    assert np.array_equal(Yp.view(np.uint32), Yu.view(np.uint32))
    v = oracle.compare_grouped(Yp, X, ti, off, q, s)
    assert v["ok"], v


def test_grouped_packed_refuses_other_kernels(dev):
    T, E, topk, N, K = 6, 4100, 3, 20, 96
    X, W, ti, off = workloads.moe_case(T, E, topk, N, K, seed=21)
    q, s = dev_words(E, N, K, 1)
    packed = binding.w4a16_grouped_pack(to_dev(q, dev), to_dev(s, dev))
    with pytest.raises(binding.W4A16Error) as err:
        binding.w4a16_gemm_grouped_packed(to_dev(X, dev), to_dev(ti, dev), to_dev(off, dev),
                                          packed, E, N)
    assert err.value.status == 2  # W4A16_ERR_SHAPE, refused before any launch
