"""GPU parity of the repack entry points against the oracle, through the C ABI:
w4a16_repack must write the oracle's pack_grouped layout (one expert) byte for
byte, and w4a16_gemm_repacked (the matrix-core decode GEMV of w4a16_gemm for
M <= 8, bit for bit its result on the public layout; otherwise the skinny
kernel or the 128 x 128 matrix-core
tile, whichever w4a16_select_path picks) must meet the tolerance on every
output."""

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
    N = qw.shape[0]
    packed = binding.w4a16_repack(to_dev(qw, dev), to_dev(sc, dev))
    out = binding.w4a16_gemm_repacked(to_dev(X, dev), packed, N, Y)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("N,K", [(1, 32), (16, 128), (17, 96), (130, 224), (300, 7168)])
def test_repack_matches_oracle_bytes(dev, N, K):
    say(f"repack bytes N={N} K={K}")
    _, W = workloads.random_case(1, N, K, seed=N * 3 + K)
    qw, sc = oracle.quantize(W)
    got = binding.w4a16_repack(to_dev(qw, dev), to_dev(sc, dev)).cpu().numpy()
    want = oracle.pack_grouped(qw[None], sc[None])
    assert got.size == binding.w4a16_repacked_bytes(N, K) == want.size
    assert np.array_equal(got, want)


SHAPES = [
    # matrix-core decode GEMV (M <= 8; past K = 8192 in several passes)
    (1, 512, 256), (2, 70, 224), (3, 33, 96), (4, 129, 512), (1, 16, 32), (2, 300, 7168),
    (5, 17, 32), (8, 100, 1056), (1, 100, 38144), (4, 64, 9344), (1, 40, 38176), (4, 20, 9376),
    # skinny kernel (9..64 rows, and above 64 rows while its rounds cost less
    # than the tile's)
    (17, 70, 160), (33, 45, 4128), (63, 33, 96), (64, 300, 7168),
    (65, 129, 224), (130, 200, 320), (300, 260, 256), (1100, 1300, 32),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_repacked_shapes(dev, M, N, K):
    say(f"repacked M={M} N={N} K={K}")
    X, W = workloads.random_case(M, N, K, seed=M * 17 + N + K)
    qw, sc = oracle.quantize(W)
    v = oracle.compare(run(X, qw, sc, dev), X, qw, sc)
    say(f"  max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


# (M, N, K): row counts of every A-operand form (1, 2, 4, 8 activation rows),
# quads per lane 1..8 (N from 17 to 7168), group counts that leave 1..3
# padding groups in the last 4-group step (G = 1, 3, 65, 66, 255) and the
# longest K (G = 256, 16 waves)
DECODE_BITWISE = [(1, 17, 32), (2, 33, 96), (3, 300, 2080), (4, 1000, 2112), (5, 129, 8160),
                  (6, 70, 8192), (7, 4096, 224), (8, 900, 7168), (1, 7168, 2048), (1, 4096, 7168)]


@pytest.mark.parametrize("M,N,K", DECODE_BITWISE)
def test_repacked_decode_matches_public_bitwise(dev, M, N, K):
    say(f"repacked decode GEMV M={M} N={N} K={K}")
    X, W = workloads.random_case(M, N, K, seed=M * 29 + N + K)
    qw, sc = oracle.quantize(W)
    got = run(X, qw, sc, dev)
    pub = binding.w4a16_gemm(to_dev(X, dev), to_dev(qw, dev), to_dev(sc, dev))
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint32), pub.cpu().numpy().view(np.uint32))
    v = oracle.compare(got, X, qw, sc)
    say(f"  max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


@pytest.mark.parametrize("name", ["tiny", "decode_gate_up", "decode_down", "verify_tree"])
def test_repacked_workloads_every_output(dev, name):
    say(f"repacked {name}")
    X, W = workloads.make(name)
    qw, sc = oracle.quantize(W)
    v = oracle.compare(run(X, qw, sc, dev), X, qw, sc)
    say(f"  max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


@pytest.mark.parametrize("M,N,K", [(2, 48, 512), (40, 48, 512)])
def test_repacked_integer_exact(dev, M, N, K):
    rng = np.random.default_rng(8 + M)
    X = rng.integers(-8, 9, (M, K)).astype(np.float32)
    nib = rng.integers(0, 16, (N, K)).astype(np.uint8)
    qw = oracle.pack(nib)
    sc = np.full((N, K // 32), np.float32(0.5), np.float32)
    Y = run(X, qw, sc, dev)
    assert np.array_equal(Y.astype(np.float64), oracle.gemm(X, qw, sc))


@pytest.mark.parametrize("M", [3, 21])
def test_repacked_guard_band_and_determinism(dev, M):
    N, K = 45, 160
    X, W = workloads.random_case(M, N, K, seed=4)
    qw, sc = oracle.quantize(W)
    pad = 4096
    buf = torch.full((pad + M * N + pad,), 0x7FC0DEAD, dtype=torch.int32, device=dev)
    Y = buf[pad:pad + M * N].view(torch.float32).view(M, N)
    a = run(X, qw, sc, dev, Y)
    host = buf.cpu().numpy().view(np.uint32)
    assert np.all(host[:pad] == 0x7FC0DEAD) and np.all(host[pad + M * N:] == 0x7FC0DEAD)
    b = run(X, qw, sc, dev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert oracle.compare(a, X, qw, sc)["ok"]


def test_repacked_nonfinite_row(dev):
    # a row holding Inf or NaN turns its outputs to NaN; the other rows are unaffected
    M, N, K = 6, 40, 256
    X, W = workloads.random_case(M, N, K, seed=12)
    X[1, 5] = np.inf
    X[4, 200] = np.nan
    qw, sc = oracle.quantize(W)
    Y = run(X, qw, sc, dev)
    assert np.all(np.isnan(Y[1])) and np.all(np.isnan(Y[4]))
    keep = [0, 2, 3, 5]
    assert oracle.compare(Y[keep], X[keep], qw, sc)["ok"]


# the 128 x 128 matrix-core tile on repacked weights (shapes w4a16_select_path
# gives to it): ragged M and N (rows padded to 16 in the layout, trailing tiles
# clamped), odd group counts (steps padded to 4 groups), and the workload
# sizes' K
TILE_SHAPES = [(2100, 1200, 160), (2200, 1290, 2080), (1700, 1600, 7168), (2300, 1300, 32),
               (2688, 1032, 96)]


@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_repacked_tile_shapes(dev, M, N, K):
    say(f"repacked tile M={M} N={N} K={K}")
    assert binding.w4a16_select_path(M, N, K) == binding.W4A16_PATH_TILE_MX
    X, W = workloads.random_case(M, N, K, seed=M + 7 * N + K)
    qw, sc = oracle.quantize(W)
    v = oracle.compare(run(X, qw, sc, dev), X, qw, sc)
    say(f"  max err/bound {v['max_ratio']:.3e}")
    assert v["ok"], v


def test_repacked_tile_integer_exact(dev):
    M, N, K = 2300, 1300, 288
    assert binding.w4a16_select_path(M, N, K) == binding.W4A16_PATH_TILE_MX
    rng = np.random.default_rng(31)
    X = rng.integers(-8, 9, (M, K)).astype(np.float32)
    nib = rng.integers(0, 16, (N, K)).astype(np.uint8)
    qw = oracle.pack(nib)
    sc = np.full((N, K // 32), np.float32(0.25), np.float32)
    Y = run(X, qw, sc, dev)
    assert np.array_equal(Y.astype(np.float64), oracle.gemm(X, qw, sc))


def test_repacked_tile_guard_band_and_nonfinite(dev):
    M, N, K = 2300, 1300, 224
    assert binding.w4a16_select_path(M, N, K) == binding.W4A16_PATH_TILE_MX
    X, W = workloads.random_case(M, N, K, seed=14)
    X[3, 17] = np.inf
    X[2299, 200] = np.nan
    qw, sc = oracle.quantize(W)
    pad = 4096
    buf = torch.full((pad + M * N + pad,), 0x7FC0DEAD, dtype=torch.int32, device=dev)
    Y = buf[pad:pad + M * N].view(torch.float32).view(M, N)
    a = run(X, qw, sc, dev, Y)
    host = buf.cpu().numpy().view(np.uint32)
    assert np.all(host[:pad] == 0x7FC0DEAD) and np.all(host[pad + M * N:] == 0x7FC0DEAD)
    assert not np.any(np.isfinite(a[3])) and not np.any(np.isfinite(a[2299]))
    keep = [m for m in range(M) if m not in (3, 2299)]
    assert oracle.compare(a[keep], X[keep], qw, sc)["ok"]
    # the same bits as the public layout's matrix-core tile
    pub = binding.w4a16_gemm_path(to_dev(X, dev), to_dev(qw, dev), to_dev(sc, dev),
                                  path=binding.W4A16_PATH_TILE_MX)
    torch.cuda.synchronize()
    assert np.array_equal(a[keep].view(np.uint32), pub.cpu().numpy()[keep].view(np.uint32))
