"""GPU parity of the small-M GEMM on packed weights (w4a16_gemm_small_packed)
against the oracle: weights packed by w4a16_grouped_pack as one expert,
1 <= M <= 64 rows (the tree-verification batches)."""

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


def run(X, qw, sc, dev, Y=None, workspace=None):
    N = qw.shape[0]
    packed = binding.w4a16_grouped_pack(to_dev(qw[None], dev), to_dev(sc[None], dev))
    out = binding.w4a16_gemm_small_packed(to_dev(X, dev), packed, N, Y, workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# M over every 16-row block count and ragged blocks; N ragged in tiles and in
# 256-column groups; K with partial steps (not a multiple of 128), one slice,
# many slices, and a long K
@pytest.mark.parametrize("M,N,K", [(64, 512, 1024), (1, 300, 7168), (5, 70, 224), (16, 256, 96),
                                   (17, 33, 512), (33, 1000, 2080), (48, 129, 4096),
                                   (63, 4100, 256), (64, 16, 32), (20, 64, 38144)])
def test_small_packed_shapes(dev, M, N, K):
    say(f"small packed M={M} N={N} K={K} ws={binding.w4a16_small_packed_workspace_bytes(M, N, K)}")
    X, W = workloads.random_case(M, N, K, seed=M * 31 + N + K)
    qw, sc = oracle.quantize(W)
    v = oracle.compare(run(X, qw, sc, dev), X, qw, sc)
    say(f"  max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


def test_small_packed_verify_tree_full(dev):
    """The tree-verification workload at full size (M=64, K=7168, N=4096),
    every output against the oracle."""
    say("small packed verify_tree")
    X, W = workloads.make("verify_tree")
    qw, sc = oracle.quantize(W)
    v = oracle.compare(run(X, qw, sc, dev), X, qw, sc)
    say(f"  max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


def test_small_packed_integer_exact(dev):
    """Small integers times codes with scale 1/2: every product and partial
    sum is exact, so the result must equal the oracle bit for bit."""
    rng = np.random.default_rng(9)
    M, N, K = 40, 96, 2048
    X = rng.integers(-8, 9, (M, K)).astype(np.float32)
    nib = rng.integers(0, 16, (N, K)).astype(np.uint8)
    qw = oracle.pack(nib)
    sc = np.full((N, K // 32), np.float32(0.5), np.float32)
    Y = run(X, qw, sc, dev)
    assert np.array_equal(Y.astype(np.float64), oracle.gemm(X, qw, sc))


def test_small_packed_rows_of_mixed_scale(dev):
    """Rows whose magnitudes differ by many powers of two, and a row of zeros:
    each row's exponent is its own."""
    rng = np.random.default_rng(12)
    M, N, K = 24, 80, 1536
    X = rng.standard_normal((M, K)).astype(np.float32)
    X *= (2.0 ** rng.integers(-30, 30, (M, 1))).astype(np.float32)
    X[7] = 0.0
    W = rng.standard_normal((N, K)).astype(np.float32)
    qw, sc = oracle.quantize(W)
    Y = run(X, qw, sc, dev)
    assert np.all(Y[7] == 0.0)
    v = oracle.compare(Y, X, qw, sc)
    assert v["ok"], v


def test_small_packed_nonfinite_row(dev):
    """A row holding Inf or NaN gives NaN in that row only."""
    rng = np.random.default_rng(13)
    M, N, K = 9, 48, 640
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[2, 100] = np.inf
    X[5, 600] = np.nan
    W = rng.standard_normal((N, K)).astype(np.float32)
    qw, sc = oracle.quantize(W)
    Y = run(X, qw, sc, dev)
    assert np.all(np.isnan(Y[2])) and np.all(np.isnan(Y[5]))
    keep = [r for r in range(M) if r not in (2, 5)]
    v = oracle.compare(Y[keep], X[keep], qw, sc)
    assert v["ok"], v


def test_small_packed_guard_band_and_determinism(dev):
    """Nothing outside Y is written, a reused dirty workspace does not matter,
    and repeated calls agree bit for bit."""
    M, N, K = 37, 75, 1184
    X, W = workloads.random_case(M, N, K, seed=6)
    qw, sc = oracle.quantize(W)
    need = binding.w4a16_small_packed_workspace_bytes(M, N, K)
    assert need > 0
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)
    pad = 4096
    buf = torch.full((pad + M * N + pad,), 0x7FC0DEAD, dtype=torch.int32, device=dev)
    Y = buf[pad:pad + M * N].view(torch.float32).view(M, N)
    a = run(X, qw, sc, dev, Y, ws)
    host = buf.cpu().numpy().view(np.uint32)
    assert np.all(host[:pad] == 0x7FC0DEAD) and np.all(host[pad + M * N:] == 0x7FC0DEAD)
    b = run(X, qw, sc, dev, None, ws)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert oracle.compare(a, X, qw, sc)["ok"]


def test_small_packed_refuses(dev):
    X = torch.zeros((65, 256), dtype=torch.float32, device=dev)
    packed = torch.zeros(binding.w4a16_grouped_pack_bytes(1, 16, 256), dtype=torch.uint8,
                         device=dev)
    with pytest.raises(binding.W4A16Error) as err:
        binding.w4a16_gemm_small_packed(X, packed, 16)
    assert err.value.status == 2  # refused before any launch
