"""GPU parity of WeightBundle.linear(): a weight with .qw/.sc files runs the
W4A16 kernels (checked against the oracle to its bound), a plain weight runs
the fp32 GEMM (checked against an fp64 product to the classical fp32 dot
product bound), both loaded from raw files through the native loader."""

import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from int4_weight_only_03_amd import binding  # noqa: E402
from int4_weight_only_03_amd.bundle import WeightBundle  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    binding.load()
    return torch.device("cuda:0")


# a decoder layer's worth of names: MLP and expert weights quantized, attention
# projection and lm_head plain (the split the pages describe)
SHAPES = {"mlp.gate_up": (256, 512), "moe.e3.down": (96, 224), "attn.q": (160, 512),
          "lm_head": (100, 96)}
QUANTIZED = ("mlp.gate_up", "moe.e3.down")


@pytest.fixture(scope="module")
def bundle_dir(tmp_path_factory):
    d = tmp_path_factory.mktemp("bundle")
    Ws = {}
    for i, (name, (N, K)) in enumerate(SHAPES.items()):
        _, W = workloads.random_case(1, N, K, seed=100 + i)
        Ws[name] = W
        if name in QUANTIZED:
            qw, sc = oracle.quantize(W)
            binding.w4a16_save_quantized(d / f"{name}.qw", d / f"{name}.sc", qw, sc)
        else:
            W.astype("<f4").tofile(d / f"{name}.f32")
    return d, Ws


def fp32_ok(Y, X, W):
    """|Y - X.W^T| <= K * 2^-24 * sum|x||w| (+ a denormal floor), elementwise."""
    X = X.astype(np.float64)
    W = W.astype(np.float64)
    ref = X @ W.T
    T = np.abs(X) @ np.abs(W).T
    tol = X.shape[1] * 2.0**-24 * T + 1e-30
    return bool(np.all(np.abs(Y - ref) <= tol)), float(np.max(np.abs(Y - ref) / tol))


@pytest.mark.parametrize("M", [1, 5, 64, 130])
def test_linear_dispatch_parity(dev, bundle_dir, M):
    d, Ws = bundle_dir
    say(f"bundle linear M={M}")
    b = WeightBundle.from_directory(d, SHAPES, device=dev)
    for i, (name, (N, K)) in enumerate(SHAPES.items()):
        X, _ = workloads.random_case(M, 1, K, seed=7 * M + i)
        Y = b.linear(name, torch.from_numpy(X).to(dev))
        torch.cuda.synchronize()
        Yh = Y.cpu().numpy()
        assert Yh.shape == (M, N)
        if name in QUANTIZED:
            qw, sc = oracle.quantize(Ws[name])
            v = oracle.compare(Yh, X, qw, sc)
            assert v["ok"], (name, v)
        else:
            ok, worst = fp32_ok(Yh, X, Ws[name])
            assert ok, (name, worst)
    assert b.calls == {"int4": 2, "fp32": 2}


def test_linear_int4_is_the_library_result(dev, bundle_dir):
    """The int4 arm returns exactly what w4a16_gemm returns on the same operands."""
    d, Ws = bundle_dir
    b = WeightBundle.from_directory(d, SHAPES, device=dev)
    X, _ = workloads.random_case(3, 1, 512, seed=9)
    Xd = torch.from_numpy(X).to(dev)
    Y1 = b.linear("mlp.gate_up", Xd)
    Y2 = binding.w4a16_gemm(Xd, b.qweight["mlp.gate_up"], b.scales["mlp.gate_up"])
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def test_linear_leading_dims_and_out(dev, bundle_dir):
    d, Ws = bundle_dir
    b = WeightBundle.from_directory(d, SHAPES, device=dev)
    X, _ = workloads.random_case(6, 1, 224, seed=11)
    Xd = torch.from_numpy(X).to(dev).view(2, 3, 224)
    out = torch.full((2, 3, 96), float("nan"), device=dev)
    Y = b.linear("moe.e3.down", Xd, out=out)
    torch.cuda.synchronize()
    assert Y.shape == (2, 3, 96) and Y.data_ptr() == out.data_ptr()
    qw, sc = oracle.quantize(Ws["moe.e3.down"])
    v = oracle.compare(out.view(6, 96).cpu().numpy(), X, qw, sc)
    assert v["ok"], v
    with pytest.raises(ValueError):
        b.linear("moe.e3.down", torch.zeros(2, 512, device=dev))
