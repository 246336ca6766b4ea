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
