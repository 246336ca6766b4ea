"""GPU parity at full size and at the accuracy limits, through the C ABI.

* The prefill workload (M = 4096, K = 7168, N = 4096): every output of every
  path against one fp64 oracle product (computed once per module).
* Ragged shapes with many 128 x 128 tiles (what w4a16_gemm runs on the
  matrix-core tile, and the fp32 tiled path's 128 x 128 kernel forced):
  clamped edge reads and masked stores, every output.
* Sign-coherent inputs (every activation >= 0 and every weight code >= 8, so
  no rounding error of a sum cancels) at K = 7168 and at the largest K each
  kernel takes, up to the library's K limit 2^17.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_only_03_amd import binding  # noqa: E402

K_MAX = 1 << 17


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


def run(X, qw, sc, path, dev):
    """One path's Y on the device (host copy); path names as in the bench."""
    Xd, Qd, Sd = to_dev(X, dev), to_dev(qw, dev), to_dev(sc, dev)
    if path == "auto":
        Y = binding.w4a16_gemm(Xd, Qd, Sd)
    elif path == "gemv":
        Y = binding.w4a16_gemm_path(Xd, Qd, Sd, path=binding.W4A16_PATH_GEMV)
    elif path == "tile":
        Y = binding.w4a16_gemm_path(Xd, Qd, Sd, path=binding.W4A16_PATH_TILE)
    elif path == "tile-mx":
        Y = binding.w4a16_gemm_path(Xd, Qd, Sd, path=binding.W4A16_PATH_TILE_MX)
    elif path == "split":
        Y = binding.w4a16_gemm_split(Xd, Qd, Sd)
    elif path == "packed":
        Y = binding.w4a16_gemm_split_packed(Xd, binding.w4a16_split_pack(Qd, Sd), qw.shape[0])
    elif path == "repacked":
        Y = binding.w4a16_gemm_repacked(Xd, binding.w4a16_repack(Qd, Sd), qw.shape[0])
    elif path == "small-packed":
        packed = binding.w4a16_grouped_pack(Qd[None], Sd[None])
        Y = binding.w4a16_gemm_small_packed(Xd, packed, qw.shape[0])
    else:
        raise ValueError(path)
    torch.cuda.synchronize()
    out = Y.cpu().numpy()
    del Xd, Qd, Sd, Y
    return out


class Ref:
    """Inputs of one problem and its fp64 oracle product, computed once."""

    def __init__(self, X, W):
        self.X = X
        self.qw, self.sc = oracle.quantize(W)
        self.Y = oracle.gemm(X, self.qw, self.sc)
        self.T = oracle.abs_gemm(X, self.qw, self.sc)

    def check(self, Y, what):
        v = oracle.compare_to(Y, self.Y, self.T)
        say(f"{what}: max err/bound {v['max_ratio']:.3e} over {v['n']} outputs")
        assert v["ok"], (what, v)


@pytest.fixture(scope="module")
def prefill():
    say("prefill oracle (M=4096 K=7168 N=4096, fp64)")
    return Ref(*workloads.make("prefill"))


@pytest.mark.parametrize("path", ["auto", "tile", "split", "packed", "repacked"])
def test_prefill_every_output(dev, prefill, path):
    assert binding.w4a16_select_path(4096, 4096, 7168) == binding.W4A16_PATH_TILE_MX
    say(f"prefill every output path={path}")
    prefill.check(run(prefill.X, prefill.qw, prefill.sc, path, dev), f"prefill {path}")


@pytest.fixture(scope="module")
def ragged_big():
    # 33 x 32 = 1056 tiles of 128 x 128: the matrix-core tile (and, forced, the
    # fp32 path's 128 x 128 kernel), with a partial last row tile (4 rows) and
    # column tile (32 columns)
    say("ragged oracle (M=4100 K=7168 N=4000, fp64)")
    return Ref(*workloads.random_case(4100, 4000, 7168, seed=41))


@pytest.mark.parametrize("path", ["auto", "tile", "split", "packed", "repacked"])
def test_ragged_wide_tiles_every_output(dev, ragged_big, path):
    say(f"ragged M=4100 N=4000 K=7168 path={path}")
    ragged_big.check(run(ragged_big.X, ragged_big.qw, ragged_big.sc, path, dev),
                     f"ragged 4100x4000x7168 {path}")


@pytest.mark.parametrize("M,N,K", [(4100, 4000, 96), (4097, 4095, 32), (8191, 2049, 224)])
@pytest.mark.parametrize("path", ["auto", "tile", "split", "repacked"])
def test_ragged_wide_tiles_short_k(dev, M, N, K, path):
    say(f"ragged M={M} N={N} K={K} path={path}")
    X, W = workloads.random_case(M, N, K, seed=M + N + K)
    ref = Ref(X, W)
    ref.check(run(X, ref.qw, ref.sc, path, dev), f"ragged {M}x{N}x{K} {path}")


# sign-coherent problems: (M, N, K, paths)
COHERENT = [
    (1, 256, 7168, ["auto", "split", "repacked"]),          # matrix-core decode GEMV
    (8, 100, 8192, ["auto", "small-packed"]),               # its longest K, 8 rows
    (64, 256, 7168, ["auto", "split", "packed", "repacked", "small-packed"]),  # skinny tiles
    (1, 64, K_MAX, ["auto", "split", "packed", "repacked", "small-packed"]),   # 64 passes
    (2, 40, K_MAX, ["auto", "repacked"]),
    (9, 64, K_MAX, ["auto", "split", "repacked", "small-packed"]),             # skinny tiles
    (130, 64, K_MAX, ["auto", "tile", "tile-mx"]),             # skinny above 64 rows, both tiles
]


@pytest.mark.parametrize("M,N,K,paths", COHERENT)
def test_sign_coherent(dev, M, N, K, paths):
    X, W = workloads.coherent_case(M, N, K, seed=M + N + K)
    ref = Ref(X, W)
    assert np.all((ref.qw.view(np.uint32) & 0x88888888) == 0x88888888)  # every code >= 8
    for path in paths:
        say(f"coherent M={M} N={N} K={K} path={path}")
        ref.check(run(X, ref.qw, ref.sc, path, dev), f"coherent {M}x{N}x{K} {path}")


def test_sign_coherent_wide_tiles(dev):
    # 32 x 16 tiles of 128 on coherent products over K = 16384: the matrix-core
    # tile, and the fp32 path's 128 x 128 kernel
    M, N, K = 4096, 2048, 16384
    assert binding.w4a16_select_path(M, N, K) == binding.W4A16_PATH_TILE_MX
    X, W = workloads.coherent_case(M, N, K, seed=9)
    say("coherent wide-tile oracle (M=4096 K=16384 N=2048, fp64)")
    ref = Ref(X, W)
    for path in ("auto", "tile"):
        say(f"coherent 4096x2048x16384 path={path}")
        ref.check(run(X, ref.qw, ref.sc, path, dev), f"coherent 4096x2048x16384 {path}")
