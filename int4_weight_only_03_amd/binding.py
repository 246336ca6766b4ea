"""Thin ctypes binding of libw4a16.so: argument marshalling only.

Every function keeps the name of the C entry point it calls.  Device buffers
are PyTorch tensors on a ROCm device (PyTorch provides memory and streams);
the arithmetic runs in the library's HIP kernels.  There is no fallback: if
the library cannot be loaded, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libw4a16.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "w4a16.h")

GROUP = 32
W4A16_OK = 0
W4A16_PATH_AUTO = 0
W4A16_PATH_GEMV = 1
W4A16_PATH_TILE = 2
W4A16_PATH_SPLIT = 3
W4A16_PATH_GEMV_FMA = 4
W4A16_PATH_TILE_MX = 5

_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({w4a16_status_str(status)})")


_SIGS = {
    "w4a16_abi_version": ([], ctypes.c_int),
    "w4a16_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "w4a16_quantize": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                        ctypes.c_int64, ctypes.c_int32], ctypes.c_int),
    "w4a16_gemm": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                    ctypes.c_void_p], ctypes.c_int),
    "w4a16_gemm_path": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                         ctypes.c_int32, ctypes.c_void_p], ctypes.c_int),
    "w4a16_select_path": ([ctypes.c_int64, ctypes.c_int64, ctypes.c_int64], ctypes.c_int),
    "w4a16_split_workspace_bytes": ([ctypes.c_int64, ctypes.c_int64, ctypes.c_int64],
                                    ctypes.c_size_t),
    "w4a16_gemm_split": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "w4a16_gemm_swiglu": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                           ctypes.c_void_p], ctypes.c_int),
    "w4a16_gemm_grouped": ([ctypes.c_void_p] * 6 + [ctypes.c_int64] * 5 + [ctypes.c_int32,
                                                                      ctypes.c_void_p],
                           ctypes.c_int),
    "w4a16_split_pack_bytes": ([ctypes.c_int64, ctypes.c_int64], ctypes.c_size_t),
    "w4a16_split_pack": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p],
                         ctypes.c_int),
    "w4a16_gemm_split_packed": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p],
                                ctypes.c_int),
    "w4a16_grouped_kernel": ([ctypes.c_int64] * 5, ctypes.c_int),
    "w4a16_gemv_kernel": ([ctypes.c_int64] * 3, ctypes.c_int),
    "w4a16_grouped_pack_bytes": ([ctypes.c_int64] * 3, ctypes.c_size_t),
    "w4a16_repacked_bytes": ([ctypes.c_int64, ctypes.c_int64, ctypes.c_int32], ctypes.c_size_t),
    "w4a16_repack": ([ctypes.c_void_p] * 3 + [ctypes.c_int64] * 2 + [ctypes.c_int32,
                                                                    ctypes.c_void_p],
                     ctypes.c_int),
    "w4a16_gemm_repacked": ([ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 +
                            [ctypes.c_int32, ctypes.c_void_p], ctypes.c_int),
    "w4a16_small_packed_workspace_bytes": ([ctypes.c_int64] * 3, ctypes.c_size_t),
    "w4a16_gemm_small_packed_noalloc": ([ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 +
                                        [ctypes.c_int32, ctypes.c_void_p], ctypes.c_int),
    "w4a16_gemm_small_packed": ([ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 +
                                [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p], ctypes.c_int),
    "w4a16_grouped_pack": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                            ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                            ctypes.c_void_p], ctypes.c_int),
    "w4a16_gemm_grouped_packed": ([ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 +
                                  [ctypes.c_int32, ctypes.c_void_p], ctypes.c_int),
    "w4a16_read_floor": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "w4a16_load_quantized": ([ctypes.c_char_p, ctypes.c_char_p, ctypes.c_int64, ctypes.c_int64,
                              ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "w4a16_save_quantized": ([ctypes.c_char_p, ctypes.c_char_p, ctypes.c_int64, ctypes.c_int64,
                              ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
}


def header_functions() -> list[str]:
    """Names of the functions include/w4a16.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_\w+)\s*\(", text)))


def load(path: str | None = None):
    """Load the library (building it first only if no build exists).

    torch is imported first: its wheel carries its own HIP runtime
    (libamdhip64.so.7, with its own ROCr), and the library's dependency on
    libamdhip64.so.7 then binds to that already-loaded copy.  Loaded before
    torch, the library would bring in the system copy, torch would add its
    own, and whichever runtime initialised the GPU second would see no device
    (launches fail with hipErrorNoDevice)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    import torch  # noqa: F401  (see above: one HIP runtime per process)
    p = path or LIB_PATH
    if not os.path.exists(p):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(p)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def w4a16_abi_version() -> int:
    return load().w4a16_abi_version()


def w4a16_status_str(status: int) -> str:
    return load().w4a16_status_str(int(status)).decode()


def w4a16_select_path(M: int, N: int, K: int) -> int:
    return load().w4a16_select_path(M, N, K)


def w4a16_quantize(W: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Host quantizer: W fp32 [N][K] -> (qweight int32 [N][K/8], scales fp32 [N][K/32])."""
    W = np.ascontiguousarray(W)
    if W.dtype != np.float32 or W.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    N, K = W.shape
    qw = np.empty((N, max(K // 8, 0)), dtype=np.int32)
    sc = np.empty((N, max(K // GROUP, 0)), dtype=np.float32)
    st = load().w4a16_quantize(W.ctypes.data, qw.ctypes.data, sc.ctypes.data, N, K, GROUP)
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_quantize")
    return qw, sc


def w4a16_load_quantized(qw_path, sc_path, N: int, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Read raw `.qw` / `.sc` files of an N x K weight into host arrays
    (qweight int32 [N][K/8], scales fp32 [N][K/32])."""
    qw = np.empty((N, max(K // 8, 0)), dtype=np.int32)
    sc = np.empty((N, max(K // GROUP, 0)), dtype=np.float32)
    st = load().w4a16_load_quantized(os.fsencode(qw_path), os.fsencode(sc_path), N, K, GROUP,
                                     qw.ctypes.data, sc.ctypes.data)
    if st != W4A16_OK:
        raise W4A16Error(st, f"w4a16_load_quantized({qw_path}, {sc_path})")
    return qw, sc


def w4a16_save_quantized(qw_path, sc_path, qweight: np.ndarray, scales: np.ndarray) -> None:
    """Write host qweight [N][K/8] int32 and scales [N][K/32] fp32 as raw `.qw` / `.sc` files."""
    qweight = np.ascontiguousarray(qweight)
    scales = np.ascontiguousarray(scales)
    if qweight.dtype != np.int32 or scales.dtype != np.float32 or qweight.ndim != 2:
        raise TypeError("qweight must be 2-D int32 and scales float32")
    N, K = qweight.shape[0], 8 * qweight.shape[1]
    if scales.shape != (N, K // GROUP):
        raise ValueError(f"scales shape {scales.shape} != {(N, K // GROUP)}")
    st = load().w4a16_save_quantized(os.fsencode(qw_path), os.fsencode(sc_path), N, K, GROUP,
                                     qweight.ctypes.data, scales.ctypes.data)
    if st != W4A16_OK:
        raise W4A16Error(st, f"w4a16_save_quantized({qw_path}, {sc_path})")


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a tensor on a ROCm device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream_ptr(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def w4a16_gemm_path(X, qweight, scales, Y=None, path: int = W4A16_PATH_AUTO, stream=None):
    """Y = X . dequant(qweight, scales)^T on the device, with the kernel path forced."""
    import torch
    X = _dev(X, torch.float32, "X")
    qweight = _dev(qweight, torch.int32, "qweight")
    scales = _dev(scales, torch.float32, "scales")
    if X.dim() != 2 or qweight.dim() != 2 or scales.dim() != 2:
        raise ValueError("X, qweight and scales must be 2-D")
    M, K = X.shape
    N = qweight.shape[0]
    if K % 8 or qweight.shape[1] != K // 8 or tuple(scales.shape) != (N, K // GROUP):
        raise ValueError(f"shapes disagree: X {tuple(X.shape)}, qweight "
                         f"{tuple(qweight.shape)}, scales {tuple(scales.shape)}")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    else:
        Y = _dev(Y, torch.float32, "Y")
        if tuple(Y.shape) != (M, N):
            raise ValueError(f"Y shape {tuple(Y.shape)} != {(M, N)}")
    st = load().w4a16_gemm_path(X.data_ptr(), qweight.data_ptr(), scales.data_ptr(),
                                Y.data_ptr(), M, N, K, GROUP, int(path),
                                _stream_ptr(stream, X.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemm_path")
    return Y


W4A16_GROUPED_MFMA = 1
W4A16_GROUPED_ROWS = 2
W4A16_GROUPED_GEMV = 3


W4A16_GEMV_MFMA = 1
W4A16_GEMV_FMA = 2
W4A16_GEMV_SKINNY = 3


def w4a16_gemv_kernel(M: int, N: int, K: int) -> int:
    """Kernel of the GEMV path for this shape (W4A16_GEMV_*), 0 if the shape is refused."""
    return load().w4a16_gemv_kernel(M, N, K)


def w4a16_grouped_kernel(T: int, R: int, E: int, N: int, K: int) -> int:
    """Kernel of w4a16_gemm_grouped for this shape (W4A16_GROUPED_*), 0 if none."""
    return load().w4a16_grouped_kernel(T, R, E, N, K)


def w4a16_grouped_pack_bytes(E: int, N: int, K: int) -> int:
    return int(load().w4a16_grouped_pack_bytes(E, N, K))


def w4a16_grouped_pack(qweight, scales, packed=None, stream=None):
    """Repack device expert weights qweight [E][N][K/8] and scales [E][N][K/32]
    for w4a16_gemm_grouped_packed (uint8 tensor)."""
    import torch
    qweight = _dev(qweight, torch.int32, "qweight")
    scales = _dev(scales, torch.float32, "scales")
    if qweight.dim() != 3 or scales.dim() != 3:
        raise ValueError("qweight and scales must be 3-D [E][N][...]")
    E, N, K8 = qweight.shape
    K = 8 * K8
    if tuple(scales.shape) != (E, N, K // GROUP):
        raise ValueError(f"shapes disagree: qweight {tuple(qweight.shape)}, "
                         f"scales {tuple(scales.shape)}")
    need = w4a16_grouped_pack_bytes(E, N, K) if N else 0
    if packed is None:
        packed = torch.empty(max(need, 1), dtype=torch.uint8, device=qweight.device)
    packed = _dev(packed, torch.uint8, "packed")
    st = load().w4a16_grouped_pack(qweight.data_ptr(), scales.data_ptr(), E, N, K, GROUP,
                                   packed.data_ptr(), packed.numel(),
                                   _stream_ptr(stream, qweight.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_grouped_pack")
    return packed


def w4a16_gemm_grouped_packed(X, token_index, expert_offsets, packed, E: int, N: int, Y=None,
                              stream=None):
    """Grouped MoE GEMM on weights from w4a16_grouped_pack (E experts of N rows)."""
    import torch
    X = _dev(X, torch.float32, "X")
    token_index = _dev(token_index, torch.int32, "token_index")
    expert_offsets = _dev(expert_offsets, torch.int32, "expert_offsets")
    packed = _dev(packed, torch.uint8, "packed")
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    T, K = X.shape
    R = token_index.numel()
    if expert_offsets.numel() != E + 1:
        raise ValueError("expert_offsets must have E + 1 entries")
    if packed.numel() < w4a16_grouped_pack_bytes(E, N, K):
        raise ValueError("packed buffer smaller than w4a16_grouped_pack_bytes(E, N, K)")
    if Y is None:
        Y = torch.empty((R, N), dtype=torch.float32, device=X.device)
    else:
        Y = _dev(Y, torch.float32, "Y")
        if tuple(Y.shape) != (R, N):
            raise ValueError(f"Y shape {tuple(Y.shape)} != {(R, N)}")
    st = load().w4a16_gemm_grouped_packed(X.data_ptr(), token_index.data_ptr(),
                                          expert_offsets.data_ptr(), packed.data_ptr(),
                                          Y.data_ptr(), T, R, E, N, K, GROUP,
                                          _stream_ptr(stream, X.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemm_grouped_packed")
    return Y


def w4a16_repacked_bytes(N: int, K: int) -> int:
    return int(load().w4a16_repacked_bytes(N, K, GROUP))


def w4a16_repack(qweight, scales, packed=None, stream=None):
    """One-time repack of device qweight [N][K/8] and scales [N][K/32] into the
    library's private layout (uint8 tensor of w4a16_repacked_bytes(N, K) bytes)."""
    import torch
    qweight = _dev(qweight, torch.int32, "qweight")
    scales = _dev(scales, torch.float32, "scales")
    if qweight.dim() != 2 or scales.dim() != 2:
        raise ValueError("qweight and scales must be 2-D")
    N, K8 = qweight.shape
    K = 8 * K8
    if tuple(scales.shape) != (N, K // GROUP):
        raise ValueError(f"shapes disagree: qweight {tuple(qweight.shape)}, "
                         f"scales {tuple(scales.shape)}")
    need = w4a16_repacked_bytes(N, K) if N else 0
    if packed is None:
        packed = torch.empty(max(need, 1), dtype=torch.uint8, device=qweight.device)
    packed = _dev(packed, torch.uint8, "packed")
    if packed.numel() < need:
        raise ValueError("packed buffer smaller than w4a16_repacked_bytes(N, K)")
    st = load().w4a16_repack(qweight.data_ptr(), scales.data_ptr(), packed.data_ptr(), N, K,
                             GROUP, _stream_ptr(stream, qweight.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_repack")
    return packed


def w4a16_gemm_repacked(X, packed, N: int, Y=None, stream=None):
    """Y = X . dequant(W)^T with W repacked by w4a16_repack (N output rows)."""
    import torch
    X = _dev(X, torch.float32, "X")
    packed = _dev(packed, torch.uint8, "packed")
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    M, K = X.shape
    if N and packed.numel() < w4a16_repacked_bytes(N, K):
        raise ValueError("packed buffer smaller than w4a16_repacked_bytes(N, K)")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    else:
        Y = _dev(Y, torch.float32, "Y")
        if tuple(Y.shape) != (M, N):
            raise ValueError(f"Y shape {tuple(Y.shape)} != {(M, N)}")
    st = load().w4a16_gemm_repacked(X.data_ptr(), packed.data_ptr(), Y.data_ptr(), M, N, K,
                                    GROUP, _stream_ptr(stream, X.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemm_repacked")
    return Y


def w4a16_small_packed_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().w4a16_small_packed_workspace_bytes(M, N, K))


def w4a16_gemm_small_packed(X, packed, N: int, Y=None, workspace=None, stream=None):
    """Small-M GEMM (M <= 64) on weights from w4a16_grouped_pack of one expert
    ([1][N][K/8] qweight, [1][N][K/32] scales), N output rows; `workspace` is a
    uint8 device tensor of at least w4a16_small_packed_workspace_bytes(M, N, K)
    bytes (allocated here if None)."""
    import torch
    X = _dev(X, torch.float32, "X")
    packed = _dev(packed, torch.uint8, "packed")
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    M, K = X.shape
    if packed.numel() < w4a16_grouped_pack_bytes(1, N, K):
        raise ValueError("packed buffer smaller than w4a16_grouped_pack_bytes(1, N, K)")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    else:
        Y = _dev(Y, torch.float32, "Y")
        if tuple(Y.shape) != (M, N):
            raise ValueError(f"Y shape {tuple(Y.shape)} != {(M, N)}")
    need = w4a16_small_packed_workspace_bytes(M, N, K) if M and N else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    workspace = _dev(workspace, torch.uint8, "workspace")
    st = load().w4a16_gemm_small_packed(X.data_ptr(), packed.data_ptr(), Y.data_ptr(), M, N, K,
                                        GROUP, workspace.data_ptr(), workspace.numel(),
                                        _stream_ptr(stream, X.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemm_small_packed")
    return Y


W4A16_ERR_SCRATCH = 7
W4A16_NOALLOC_SCRATCH_BYTES = 64 << 20


def w4a16_gemm_small_packed_noalloc(X, packed, N: int, Y=None, stream=None):
    """w4a16_gemm_small_packed with the split-K partials in the library's fixed
    device scratch (no workspace, nothing allocated by the library)."""
    import torch
    X = _dev(X, torch.float32, "X")
    packed = _dev(packed, torch.uint8, "packed")
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    M, K = X.shape
    if packed.numel() < w4a16_grouped_pack_bytes(1, N, K):
        raise ValueError("packed buffer smaller than w4a16_grouped_pack_bytes(1, N, K)")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    else:
        Y = _dev(Y, torch.float32, "Y")
        if tuple(Y.shape) != (M, N):
            raise ValueError(f"Y shape {tuple(Y.shape)} != {(M, N)}")
    st = load().w4a16_gemm_small_packed_noalloc(X.data_ptr(), packed.data_ptr(), Y.data_ptr(),
                                                M, N, K, GROUP, _stream_ptr(stream, X.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemm_small_packed_noalloc")
    return Y


def w4a16_split_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().w4a16_split_workspace_bytes(M, N, K))


def _check_operands(X, qweight, scales, Y, allocate=True):
    import torch
    X = _dev(X, torch.float32, "X")
    qweight = _dev(qweight, torch.int32, "qweight")
    scales = _dev(scales, torch.float32, "scales")
    if X.dim() != 2 or qweight.dim() != 2 or scales.dim() != 2:
        raise ValueError("X, qweight and scales must be 2-D")
    M, K = X.shape
    N = qweight.shape[0]
    if K % 8 or qweight.shape[1] != K // 8 or tuple(scales.shape) != (N, K // GROUP):
        raise ValueError(f"shapes disagree: X {tuple(X.shape)}, qweight "
                         f"{tuple(qweight.shape)}, scales {tuple(scales.shape)}")
    if Y is None:
        if allocate:
            Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    else:
        Y = _dev(Y, torch.float32, "Y")
        if tuple(Y.shape) != (M, N):
            raise ValueError(f"Y shape {tuple(Y.shape)} != {(M, N)}")
    return X, qweight, scales, Y, M, N, K


def w4a16_gemm_split(X, qweight, scales, Y=None, workspace=None, stream=None):
    """Split-precision path; `workspace` is a uint8 device tensor of at least
    w4a16_split_workspace_bytes(M, N, K) bytes (allocated here if None)."""
    import torch
    X, qweight, scales, Y, M, N, K = _check_operands(X, qweight, scales, Y)
    need = w4a16_split_workspace_bytes(M, N, K) if M and N else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    workspace = _dev(workspace, torch.uint8, "workspace")
    st = load().w4a16_gemm_split(X.data_ptr(), qweight.data_ptr(), scales.data_ptr(),
                                 Y.data_ptr(), M, N, K, GROUP, workspace.data_ptr(),
                                 workspace.numel(), _stream_ptr(stream, X.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemm_split")
    return Y


def w4a16_gemm_swiglu(X, qweight, scales, Y=None, stream=None):
    """Y[M][F] = silu(X . gate^T) * (X . up^T); qweight/scales hold 2F rows (gate, then up)."""
    import torch
    X, qweight, scales, _, M, N2, K = _check_operands(X, qweight, scales, None, allocate=False)
    if N2 % 2:
        raise ValueError("the gate/up matrix needs an even number of rows")
    F = N2 // 2
    if Y is None:
        Y = torch.empty((M, F), dtype=torch.float32, device=X.device)
    else:
        Y = _dev(Y, torch.float32, "Y")
        if tuple(Y.shape) != (M, F):
            raise ValueError(f"Y shape {tuple(Y.shape)} != {(M, F)}")
    st = load().w4a16_gemm_swiglu(X.data_ptr(), qweight.data_ptr(), scales.data_ptr(),
                                  Y.data_ptr(), M, F, K, GROUP, _stream_ptr(stream, X.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemm_swiglu")
    return Y


def w4a16_gemm_grouped(X, token_index, expert_offsets, qweight, scales, Y=None, stream=None):
    """Grouped MoE GEMM: Y[r] = X[token_index[r]] . dequant(W_e)^T for the expert e
    owning slot r; qweight [E][N][K/8], scales [E][N][K/32], offsets [E+1]."""
    import torch
    X = _dev(X, torch.float32, "X")
    token_index = _dev(token_index, torch.int32, "token_index")
    expert_offsets = _dev(expert_offsets, torch.int32, "expert_offsets")
    qweight = _dev(qweight, torch.int32, "qweight")
    scales = _dev(scales, torch.float32, "scales")
    if X.dim() != 2 or qweight.dim() != 3 or scales.dim() != 3:
        raise ValueError("X must be 2-D, qweight and scales 3-D [E][N][...]")
    T, K = X.shape
    E, N, K8 = qweight.shape
    R = token_index.numel()
    if K8 * 8 != K or tuple(scales.shape) != (E, N, K // GROUP) or expert_offsets.numel() != E + 1:
        raise ValueError("shapes disagree")
    if Y is None:
        Y = torch.empty((R, N), dtype=torch.float32, device=X.device)
    else:
        Y = _dev(Y, torch.float32, "Y")
        if tuple(Y.shape) != (R, N):
            raise ValueError(f"Y shape {tuple(Y.shape)} != {(R, N)}")
    st = load().w4a16_gemm_grouped(X.data_ptr(), token_index.data_ptr(),
                                   expert_offsets.data_ptr(), qweight.data_ptr(),
                                   scales.data_ptr(), Y.data_ptr(), T, R, E, N, K, GROUP,
                                   _stream_ptr(stream, X.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemm_grouped")
    return Y


def w4a16_split_pack_bytes(N: int, K: int) -> int:
    return int(load().w4a16_split_pack_bytes(N, K))


def w4a16_split_pack(qweight, scales, packed=None, stream=None):
    """Repack device qweight/scales for w4a16_gemm_split_packed (uint8 tensor)."""
    import torch
    qweight = _dev(qweight, torch.int32, "qweight")
    scales = _dev(scales, torch.float32, "scales")
    N, K8 = qweight.shape
    K = 8 * K8
    if tuple(scales.shape) != (N, K // GROUP):
        raise ValueError(f"shapes disagree: qweight {tuple(qweight.shape)}, "
                         f"scales {tuple(scales.shape)}")
    need = w4a16_split_pack_bytes(N, K) if N else 0
    if packed is None:
        packed = torch.empty(max(need, 1), dtype=torch.uint8, device=qweight.device)
    packed = _dev(packed, torch.uint8, "packed")
    st = load().w4a16_split_pack(qweight.data_ptr(), scales.data_ptr(), N, K, GROUP,
                                 packed.data_ptr(), packed.numel(),
                                 _stream_ptr(stream, qweight.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_split_pack")
    return packed


def w4a16_gemm_split_packed(X, packed, N: int, Y=None, workspace=None, stream=None):
    """Split path on weights from w4a16_split_pack (N rows); workspace as for
    w4a16_gemm_split (allocated here if None)."""
    import torch
    X = _dev(X, torch.float32, "X")
    packed = _dev(packed, torch.uint8, "packed")
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    M, K = X.shape
    if packed.numel() < w4a16_split_pack_bytes(N, K):
        raise ValueError("packed buffer smaller than w4a16_split_pack_bytes(N, K)")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    else:
        Y = _dev(Y, torch.float32, "Y")
        if tuple(Y.shape) != (M, N):
            raise ValueError(f"Y shape {tuple(Y.shape)} != {(M, N)}")
    need = w4a16_split_workspace_bytes(M, N, K) if M and N else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    workspace = _dev(workspace, torch.uint8, "workspace")
    st = load().w4a16_gemm_split_packed(X.data_ptr(), packed.data_ptr(), Y.data_ptr(), M, N, K,
                                        GROUP, workspace.data_ptr(), workspace.numel(),
                                        _stream_ptr(stream, X.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gemm_split_packed")
    return Y


def w4a16_gemm(X, qweight, scales, Y=None, stream=None):
    """Y = X . dequant(qweight, scales)^T on the device (path chosen by the library)."""
    return w4a16_gemm_path(X, qweight, scales, Y, W4A16_PATH_AUTO, stream)


def w4a16_read_floor(buffers, sink, threads: int = 256, loads: int = 4, stream=None):
    """Measurement helper: one launch streaming the device tensors in `buffers`
    (up to 4, 16-byte aligned, sizes multiples of 16 bytes); `sink` is a device
    tensor of at least 4 bytes."""
    import torch
    if not 1 <= len(buffers) <= 4:
        raise ValueError("1 to 4 buffers")
    ptrs = (ctypes.c_void_p * len(buffers))(*[b.data_ptr() for b in buffers])
    sizes = (ctypes.c_int64 * len(buffers))(*[b.numel() * b.element_size() for b in buffers])
    st = load().w4a16_read_floor(ptrs, sizes, len(buffers), threads, loads, sink.data_ptr(),
                                 _stream_ptr(stream, sink.device))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_read_floor")
