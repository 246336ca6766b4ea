"""GPU parity of the fused gate/up SwiGLU (w4a16_gemm_swiglu) against the oracle.

Y[m][j] = silu(X[m] . gate_j) * (X[m] . up_j), W rows 0..F-1 gate, F..2F-1 up;
checked elementwise with the oracle's propagated bound (compare_swiglu).
"""

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


def run(X, qw, sc, dev, Y=None):
    out = binding.w4a16_gemm_swiglu(to_dev(X, dev), to_dev(qw, dev), to_dev(sc, dev), Y)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("M,F,K", [(1, 1, 32), (1, 33, 96), (2, 70, 224), (1, 300, 256),
                                   (1, 2048, 7168), (2, 64, 2048), (3, 70, 224), (5, 128, 512),
                                   (64, 96, 2048), (1, 129, 16384 + 32),
                                   # the matrix-core GEMV with 4 and 8 activation rows
                                   (4, 257, 7168), (8, 2048, 7168), (7, 33, 2080)])
def test_swiglu_shapes(dev, M, F, K):
    say(f"swiglu M={M} F={F} K={K}")
    X, W = workloads.random_case(M, 2 * F, K, seed=M * 7 + F * 11 + K)
    qw, sc = oracle.quantize(W)
    v = oracle.compare_swiglu(run(X, qw, sc, dev), X, qw, sc)
    say(f"  max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


def test_swiglu_decode_gate_up_workload(dev):
    # the decode gate+up matrix (2 x 2048 rows, K = 7168) as its own workload
    X, W = workloads.make("decode_gate_up")
    qw, sc = oracle.quantize(W)
    v = oracle.compare_swiglu(run(X, qw, sc, dev), X, qw, sc)
    say(f"decode_gate_up swiglu: max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


def test_swiglu_no_write_outside_y_and_deterministic(dev):
    M, F, K = 2, 45, 96
    X, W = workloads.random_case(M, 2 * F, K, seed=4)
    qw, sc = oracle.quantize(W)
    pad = 4096
    buf = torch.full((pad + M * F + pad,), 0x7FC0DEAD, dtype=torch.int32, device=dev)
    Y = buf[pad:pad + M * F].view(torch.float32).view(M, F)
    a = run(X, qw, sc, dev, Y)
    host = buf.cpu().numpy().view(np.uint32)
    assert np.all(host[:pad] == 0x7FC0DEAD) and np.all(host[pad + M * F:] == 0x7FC0DEAD)
    b = run(X, qw, sc, dev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert oracle.compare_swiglu(a, X, qw, sc)["ok"]


def test_swiglu_extreme_gates(dev):
    # gates far into both tails of silu: exp overflow / underflow paths
    rng = np.random.default_rng(3)
    M, F, K = 1, 64, 64
    X = np.ones((M, K), np.float32)
    nib = np.full((2 * F, K), 8, np.uint8)
    nib[:F, :] = np.where(np.arange(F)[:, None] % 2 == 0, 15, 0)  # gate +/- large
    nib[F:, :] = rng.integers(0, 16, (F, K)).astype(np.uint8)
    qw = oracle.pack(nib)
    sc = np.full((2 * F, K // 32), np.float32(8.0), np.float32)  # |g| up to 64*8*8
    v = oracle.compare_swiglu(run(X, qw, sc, dev), X, qw, sc)
    assert v["ok"], v


# Above 8 rows the fused form of the skinny kernel: 16-row tiles of X against
# the gate and up tiles of 32 outputs (16 when that leaves under 256
# workgroups); ragged rows, outputs and groups (K % 128 != 0), and the
# decode MLP at batches of 16 and 64.
SKINNY_SW = [(9, 40, 96), (9, 1, 32), (16, 2048, 7168), (17, 5000, 256), (33, 33, 2080),
             (64, 2048, 7168), (65, 129, 224), (130, 300, 4160), (700, 96, 128),
             (2050, 70, 96)]


@pytest.mark.parametrize("M,F,K", SKINNY_SW)
def test_swiglu_above_eight_rows(dev, M, F, K):
    say(f"swiglu (skinny) M={M} F={F} K={K}")
    X, W = workloads.random_case(M, 2 * F, K, seed=3 * M + 5 * F + K)
    qw, sc = oracle.quantize(W)
    v = oracle.compare_swiglu(run(X, qw, sc, dev), X, qw, sc)
    say(f"  max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


def test_swiglu_above_eight_rows_no_write_outside_y(dev):
    M, F, K = 21, 45, 160
    X, W = workloads.random_case(M, 2 * F, K, seed=12)
    qw, sc = oracle.quantize(W)
    pad = 4096
    buf = torch.full((pad + M * F + pad,), 0x7FC0DEAD, dtype=torch.int32, device=dev)
    Y = buf[pad:pad + M * F].view(torch.float32).view(M, F)
    a = run(X, qw, sc, dev, Y)
    host = buf.cpu().numpy().view(np.uint32)
    assert np.all(host[:pad] == 0x7FC0DEAD) and np.all(host[pad + M * F:] == 0x7FC0DEAD)
    b = run(X, qw, sc, dev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert oracle.compare_swiglu(a, X, qw, sc)["ok"]


def test_swiglu_above_eight_rows_extreme_gates(dev):
    # the tails of silu through the skinny epilogue, 12 rows of X at scales
    # 2^-4 .. 2^7 (per-row limb exponents)
    rng = np.random.default_rng(5)
    M, F, K = 12, 64, 128
    X = (np.ones((M, K)) * (2.0 ** np.arange(-4, 8))[:, None]).astype(np.float32)
    nib = np.full((2 * F, K), 8, np.uint8)
    nib[:F, :] = np.where(np.arange(F)[:, None] % 2 == 0, 15, 0)
    nib[F:, :] = rng.integers(0, 16, (F, K)).astype(np.uint8)
    qw = oracle.pack(nib)
    sc = np.full((2 * F, K // 32), np.float32(8.0), np.float32)
    v = oracle.compare_swiglu(run(X, qw, sc, dev), X, qw, sc)
    assert v["ok"], v


@pytest.mark.parametrize("M,F,K", [(5, 2048, 4096), (8, 2050, 4128), (6, 3000, 7168)])
def test_swiglu_five_to_eight_rows_on_large_weights(dev, M, F, K):
    # 5..8 rows on a 2F x K matrix of at least 4096 x 4096 take the skinny
    # kernel's fused form, as w4a16_gemm does on such weights
    assert binding.w4a16_gemv_kernel(M, 2 * F, K) == binding.W4A16_GEMV_SKINNY
    X, W = workloads.random_case(M, 2 * F, K, seed=M * 13 + F + K)
    qw, sc = oracle.quantize(W)
    v = oracle.compare_swiglu(run(X, qw, sc, dev), X, qw, sc)
    say(f"swiglu (skinny) {M}x{F}x{K}: max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v
