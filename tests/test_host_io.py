"""Raw .qw/.sc weight files (w4a16_load_quantized / w4a16_save_quantized) and
the WeightBundle dispatch rule, on the host (no GPU).

The files are bare little-endian arrays: the reference for their bytes is
numpy's own raw writer (`tofile`), not the library.
"""

import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from int4_weight_only_03_amd import binding  # noqa: E402
from int4_weight_only_03_amd.bundle import WeightBundle  # noqa: E402

W4A16_ERR_ARG, W4A16_ERR_SHAPE, W4A16_ERR_NONFINITE, W4A16_ERR_IO = 1, 2, 4, 6


def words(N, K, seed):
    rng = np.random.default_rng(seed)
    qw = rng.integers(-2**31, 2**31, size=(N, K // 8), dtype=np.int64).astype(np.int32)
    sc = rng.uniform(0.0, 0.5, size=(N, K // 32)).astype(np.float32)
    return qw, sc


def raw_load(qp, sp, N, K, group=32):
    qw = np.zeros((max(N, 1), max(K // 8, 1)), np.int32)
    sc = np.zeros((max(N, 1), max(K // 32, 1)), np.float32)
    st = binding.load().w4a16_load_quantized(os.fsencode(qp), os.fsencode(sp), N, K, group,
                                             qw.ctypes.data, sc.ctypes.data)
    return st, qw, sc


@pytest.mark.parametrize("N,K", [(1, 32), (7, 96), (64, 7168), (3, 4096 + 32)])
def test_load_reads_numpy_raw_files(tmp_path, N, K):
    qw, sc = words(N, K, N + K)
    qw.astype("<i4").tofile(tmp_path / "w.qw")
    sc.astype("<f4").tofile(tmp_path / "w.sc")
    q2, s2 = binding.w4a16_load_quantized(tmp_path / "w.qw", tmp_path / "w.sc", N, K)
    assert np.array_equal(q2, qw) and np.array_equal(s2.view(np.uint32), sc.view(np.uint32))


def test_save_writes_numpy_raw_bytes(tmp_path):
    N, K = 9, 224
    qw, sc = words(N, K, 3)
    binding.w4a16_save_quantized(tmp_path / "a.qw", tmp_path / "a.sc", qw, sc)
    qw.astype("<i4").tofile(tmp_path / "b.qw")
    sc.astype("<f4").tofile(tmp_path / "b.sc")
    for ext in ("qw", "sc"):
        assert (tmp_path / f"a.{ext}").read_bytes() == (tmp_path / f"b.{ext}").read_bytes()
    assert os.path.getsize(tmp_path / "a.qw") == N * K // 2
    assert os.path.getsize(tmp_path / "a.sc") == N * K // 8


def test_empty_weight(tmp_path):
    qw, sc = words(0, 64, 1)
    binding.w4a16_save_quantized(tmp_path / "e.qw", tmp_path / "e.sc", qw, sc)
    q2, s2 = binding.w4a16_load_quantized(tmp_path / "e.qw", tmp_path / "e.sc", 0, 64)
    assert q2.shape == (0, 8) and s2.shape == (0, 2)


@pytest.mark.parametrize("cut", [-1, 1, -4])
def test_wrong_size_is_io_error(tmp_path, cut):
    N, K = 4, 64
    qw, sc = words(N, K, 2)
    data = qw.astype("<i4").tobytes()
    (tmp_path / "w.qw").write_bytes(data[:cut] if cut < 0 else data + b"\0" * cut)
    sc.astype("<f4").tofile(tmp_path / "w.sc")
    st, _, _ = raw_load(tmp_path / "w.qw", tmp_path / "w.sc", N, K)
    assert st == W4A16_ERR_IO
    # right .qw, .sc of another weight's size
    qw.astype("<i4").tofile(tmp_path / "w.qw")
    words(N + 1, K, 2)[1].astype("<f4").tofile(tmp_path / "w.sc")
    assert raw_load(tmp_path / "w.qw", tmp_path / "w.sc", N, K)[0] == W4A16_ERR_IO


def test_missing_or_directory_is_io_error(tmp_path):
    N, K = 2, 32
    qw, sc = words(N, K, 5)
    qw.tofile(tmp_path / "w.qw")
    assert raw_load(tmp_path / "w.qw", tmp_path / "nope.sc", N, K)[0] == W4A16_ERR_IO
    assert raw_load(tmp_path, tmp_path / "w.qw", N, K)[0] == W4A16_ERR_IO
    with pytest.raises(binding.W4A16Error) as e:
        binding.w4a16_load_quantized(tmp_path / "w.qw", tmp_path / "nope.sc", N, K)
    assert e.value.status == W4A16_ERR_IO
    st = binding.load().w4a16_save_quantized(os.fsencode(tmp_path / "no" / "x.qw"),
                                             os.fsencode(tmp_path / "no" / "x.sc"), N, K, 32,
                                             qw.ctypes.data, sc.ctypes.data)
    assert st == W4A16_ERR_IO


def test_nonfinite_scale(tmp_path):
    N, K = 3, 64
    qw, sc = words(N, K, 6)
    for bad in (np.nan, np.inf, -np.inf):
        s = sc.copy()
        s[1, 1] = bad
        qw.tofile(tmp_path / "w.qw")
        s.tofile(tmp_path / "w.sc")
        assert raw_load(tmp_path / "w.qw", tmp_path / "w.sc", N, K)[0] == W4A16_ERR_NONFINITE
        with pytest.raises(binding.W4A16Error):
            binding.w4a16_save_quantized(tmp_path / "z.qw", tmp_path / "z.sc", qw, s)
        assert not (tmp_path / "z.qw").exists()  # checked before anything is written


def test_argument_errors(tmp_path):
    lib = binding.load()
    qw, sc = words(2, 64, 7)
    qw.tofile(tmp_path / "w.qw")
    sc.tofile(tmp_path / "w.sc")
    q, s = os.fsencode(tmp_path / "w.qw"), os.fsencode(tmp_path / "w.sc")
    buf_q, buf_s = np.zeros(64, np.int32), np.zeros(64, np.float32)
    pq, ps = buf_q.ctypes.data, buf_s.ctypes.data
    assert lib.w4a16_load_quantized(q, s, 2, 64, 16, pq, ps) == W4A16_ERR_ARG
    assert lib.w4a16_load_quantized(q, s, -1, 64, 32, pq, ps) == W4A16_ERR_ARG
    assert lib.w4a16_load_quantized(q, s, 2, 0, 32, pq, ps) == W4A16_ERR_ARG
    assert lib.w4a16_load_quantized(q, s, 2, 48, 32, pq, ps) == W4A16_ERR_SHAPE
    assert lib.w4a16_load_quantized(None, s, 2, 64, 32, pq, ps) == W4A16_ERR_ARG
    assert lib.w4a16_load_quantized(q, s, 2, 64, 32, None, ps) == W4A16_ERR_ARG
    assert lib.w4a16_save_quantized(q, None, 2, 64, 32, pq, ps) == W4A16_ERR_ARG
    assert lib.w4a16_load_quantized(q, s, 2, 64, 32, pq, ps) == 0
    assert binding.w4a16_status_str(W4A16_ERR_IO).startswith("weight file")


def make_bundle_dir(path, seed=0):
    """Two quantized weights, one plain one, one name with both forms."""
    os.makedirs(path, exist_ok=True)
    rng = np.random.default_rng(seed)
    shapes = {"mlp.up": (48, 96), "moe.e0": (8, 64), "attn.q": (16, 96), "both": (4, 32)}
    for i, name in enumerate(("mlp.up", "moe.e0", "both")):
        qw, sc = words(*shapes[name], seed=seed * 10 + i)
        binding.w4a16_save_quantized(path / f"{name}.qw", path / f"{name}.sc", qw, sc)
    for name in ("attn.q", "both"):
        rng.standard_normal(shapes[name]).astype("<f4").tofile(path / f"{name}.f32")
    return shapes


def test_bundle_dispatch_rule(tmp_path):
    shapes = make_bundle_dir(tmp_path)
    b = WeightBundle.from_directory(tmp_path, shapes, device="cpu")
    assert b.is_int4("mlp.up") and b.is_int4("moe.e0") and b.is_int4("both")
    assert not b.is_int4("attn.q")
    assert b.shape("mlp.up") == (48, 96) and b.shape("attn.q") == (16, 96)
    with pytest.raises(KeyError):
        b.is_int4("lm_head")
    # no host path: linear needs device tensors
    with pytest.raises(TypeError):
        b.linear("mlp.up", torch.zeros(1, 96))
    with pytest.raises(TypeError):
        b.linear("attn.q", torch.zeros(1, 96))


def test_bundle_round_trip_and_file_errors(tmp_path):
    shapes = make_bundle_dir(tmp_path / "a")
    b = WeightBundle.from_directory(tmp_path / "a", shapes, device="cpu")
    b.save(tmp_path / "b")
    for name in ("mlp.up", "moe.e0", "both"):
        for ext in ("qw", "sc"):
            assert (tmp_path / "a" / f"{name}.{ext}").read_bytes() == \
                (tmp_path / "b" / f"{name}.{ext}").read_bytes()
    assert (tmp_path / "a" / "attn.q.f32").read_bytes() == \
        (tmp_path / "b" / "attn.q.f32").read_bytes()
    assert not (tmp_path / "b" / "both.f32").exists()
    # a .qw without its .sc is an error, not an fp32 fallback
    os.remove(tmp_path / "a" / "moe.e0.sc")
    with pytest.raises(binding.W4A16Error):
        WeightBundle.from_directory(tmp_path / "a", shapes, device="cpu")
    with pytest.raises(FileNotFoundError):
        WeightBundle.from_directory(tmp_path / "a", {"lm_head": (4, 32)}, device="cpu")
    with pytest.raises(ValueError):
        WeightBundle.from_directory(tmp_path / "a", {"attn.q": (16, 64)}, device="cpu")
    with pytest.raises(binding.W4A16Error):  # the .qw is 48 x 96, not 48 x 64
        WeightBundle.from_directory(tmp_path / "b", {"mlp.up": (48, 64)}, device="cpu")
