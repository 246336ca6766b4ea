"""Host-side tests of the C-ABI library (no GPU is touched).

* the library loads and exports every function include/w4a16.h declares;
* the host quantizer is bit-exact with the oracle (one correct result);
* argument errors come back synchronously with the documented codes, before
  any launch: these calls use fake device addresses that are never dereferenced.
"""

import ctypes
import os
import sys

import numpy as np
import pytest

import oracle
import workloads
from int4_weight_only_03_amd import binding

OK, ARG, SHAPE, ALIGN, NONFINITE, HIP, IO, SCRATCH = 0, 1, 2, 3, 4, 5, 6, 7


def test_exports_every_declared_symbol(lib):
    names = binding.header_functions()
    assert {"w4a16_gemm", "w4a16_quantize", "w4a16_gemm_path", "w4a16_status_str",
            "w4a16_abi_version", "w4a16_select_path", "w4a16_gemm_split",
            "w4a16_split_workspace_bytes", "w4a16_split_pack", "w4a16_split_pack_bytes",
            "w4a16_gemm_split_packed", "w4a16_gemm_swiglu", "w4a16_gemm_grouped",
            "w4a16_repacked_bytes", "w4a16_repack", "w4a16_gemm_repacked"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.w4a16_abi_version() == 2


def test_status_strings(lib):
    seen = set()
    for code in (OK, ARG, SHAPE, ALIGN, NONFINITE, HIP, IO, SCRATCH):
        text = binding.w4a16_status_str(code)
        assert text and text not in seen
        seen.add(text)
    assert binding.w4a16_status_str(99) == "unknown status"


def test_gemv_kernel(lib):
    # matrix-core decode GEMV for M <= 8 at any K; the skinny matrix-core
    # kernel from 9 rows on; the fp32 FMA GEMV is never the automatic choice
    assert binding.w4a16_gemv_kernel(1, 4096, 7168) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(2, 7, 8192) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(1, 64, 8192 + 32) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(2, 64, 1 << 17) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(3, 64, 8192 + 32) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(8, 64, 1 << 17) == binding.W4A16_GEMV_MFMA
    # 5..8 rows on weights of at least 4096 x 4096: the skinny kernel
    assert binding.w4a16_gemv_kernel(4, 4096, 7168) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(5, 4096, 4096) == binding.W4A16_GEMV_SKINNY
    assert binding.w4a16_gemv_kernel(8, 14336, 4096) == binding.W4A16_GEMV_SKINNY
    assert binding.w4a16_gemv_kernel(8, 4095, 7168) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(8, 4096, 4064) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(4, 64, 256) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(8, 64, 256) == binding.W4A16_GEMV_MFMA
    assert binding.w4a16_gemv_kernel(9, 64, 256) == binding.W4A16_GEMV_SKINNY
    assert binding.w4a16_gemv_kernel(64, 4096, 7168) == binding.W4A16_GEMV_SKINNY
    assert binding.w4a16_gemv_kernel(65, 64, 256) == binding.W4A16_GEMV_SKINNY
    assert binding.w4a16_gemv_kernel(4096, 4096, 7168) == binding.W4A16_GEMV_SKINNY
    assert binding.w4a16_gemv_kernel(0, 64, 256) == 0
    assert binding.w4a16_gemv_kernel(1, 64, 250) == 0
    assert binding.w4a16_gemv_kernel(1, 0, 256) == 0


def skinny_cost(M, N):
    # rounds of 256 workgroups of 16 x 16 NT outputs, NT the widest of 4, 2, 1
    # that leaves at least 256 workgroups, each weighted by NT
    tm = -(-M // 16)
    nt = next((t for t in (4, 2) if -(-N // (16 * t)) * tm >= 256), 1)
    return -(-(tm * -(-N // (16 * nt))) // 256) * nt


def tile_cost(M, N):
    # rounds of 256 tiles of 128 x 128, each weighted by 33
    return -(-(-(-M // 128) * -(-N // 128)) // 256) * 33


def test_select_path(lib):
    # the decode/verify path for M <= 64; above, the skinny kernel (still the
    # GEMV path) while its weighted rounds cost no more than the matrix-core
    # tile's; the fp32 tiled path is never the automatic choice
    GEMV, TMX = binding.W4A16_PATH_GEMV, binding.W4A16_PATH_TILE_MX
    for M in (1, 4, 5, 8, 9, 17, 64):
        assert binding.w4a16_select_path(M, 4096, 7168) == GEMV
    assert binding.w4a16_select_path(5, 4096, 8192 + 32) == GEMV
    # N = 4096: 512 rows cost 8 skinny rounds x 4 = 32 <= 33; 513 rows 9 x 4 = 36
    for M, want in ((65, GEMV), (256, GEMV), (257, GEMV), (512, GEMV), (513, TMX),
                    (4096, TMX)):
        assert binding.w4a16_select_path(M, 4096, 7168) == want, M
    # N = 14336: 144 rows cost 8 x 4 = 32, 145 rows 9 x 4 = 36, against one
    # round of 224 tiles
    assert binding.w4a16_select_path(144, 14336, 4096) == GEMV
    assert binding.w4a16_select_path(145, 14336, 4096) == TMX
    # narrow N: the skinny kernel at every M measured
    assert binding.w4a16_select_path(768, 2048, 7168) == GEMV
    assert binding.w4a16_select_path(65, 12161, 7168) == GEMV
    assert binding.w4a16_select_path(1 << 24, 1 << 30, 32) == TMX
    # extents the GEMM refuses or treats as no-ops still get an answer
    assert binding.w4a16_select_path(0, 4096, 7168) == GEMV
    assert binding.w4a16_select_path(1 << 40, 4096, 7168) == TMX
    assert binding.w4a16_select_path(4096, 1 << 40, 7168) == TMX
    # the rule itself over a grid of shapes
    for M in (65, 100, 128, 200, 300, 500, 1000, 3000):
        for N in (16, 100, 1024, 3000, 7168, 20000):
            want = GEMV if skinny_cost(M, N) <= tile_cost(M, N) else TMX
            assert binding.w4a16_select_path(M, N, 4096) == want, (M, N)


# ------------------------------------------------------------------ quantize

@pytest.mark.parametrize("name", ["tiny", "decode_down", "decode_gate_up", "verify_tree",
                                  "prefill"])
def test_quantize_bit_exact_with_oracle(lib, name):
    W = workloads.make_w(name)
    qa, sa = binding.w4a16_quantize(W)
    qb, sb = oracle.quantize(W)
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
    assert np.array_equal(qa, qb)


def test_quantize_edge_groups(lib):
    rng = np.random.default_rng(17)
    W = (0.02 * rng.standard_normal((12, 256))).astype(np.float32)
    W[0, :32] = 0.0                                        # all-zero group
    W[1, 32:64] = -0.0                                     # negative zeros
    W[2, 64:96] = np.float32(2.0 ** -149)                  # scale underflows to 0
    W[3, :32] = np.ldexp(rng.standard_normal(32), -140).astype(np.float32)  # subnormal scale
    W[4, :32] = np.arange(32, dtype=np.float32) - 16.0     # 2.5-style ties at scale 16/7
    W[5, :32] = np.float32(3.0e38) * np.sign(rng.standard_normal(32)).astype(np.float32)
    W[6, :8] = [7, 3.5, 2.5, -2.5, 0.5, 1.5, -0.5, -7]     # exact ties, scale 1
    W[7] = np.float32(1e-3) * np.sign(rng.standard_normal(256)).astype(np.float32)
    qa, sa = binding.w4a16_quantize(W)
    qb, sb = oracle.quantize(W)
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
    assert np.array_equal(qa, qb)


def test_quantize_errors_leave_outputs_untouched(lib):
    W = np.zeros((2, 64), np.float32)
    W[1, 40] = np.nan
    qw = np.full((2, 8), 7, np.int32)
    sc = np.full((2, 2), 5.0, np.float32)
    st = lib.w4a16_quantize(W.ctypes.data, qw.ctypes.data, sc.ctypes.data, 2, 64, 32)
    assert st == NONFINITE
    assert np.all(qw == 7) and np.all(sc == 5.0)
    W[1, 40] = -np.inf
    assert lib.w4a16_quantize(W.ctypes.data, qw.ctypes.data, sc.ctypes.data, 2, 64, 32) == NONFINITE
    W[1, 40] = 0.0
    assert lib.w4a16_quantize(W.ctypes.data, qw.ctypes.data, sc.ctypes.data, 2, 48, 32) == SHAPE
    assert lib.w4a16_quantize(W.ctypes.data, qw.ctypes.data, sc.ctypes.data, 2, 64, 16) == ARG
    assert lib.w4a16_quantize(W.ctypes.data, qw.ctypes.data, sc.ctypes.data, -1, 64, 32) == ARG
    assert lib.w4a16_quantize(W.ctypes.data, qw.ctypes.data, sc.ctypes.data, 2, 0, 32) == ARG
    assert lib.w4a16_quantize(None, qw.ctypes.data, sc.ctypes.data, 2, 64, 32) == ARG
    assert lib.w4a16_quantize(None, None, None, 0, 64, 32) == OK
    assert np.all(qw == 7) and np.all(sc == 5.0)
    with pytest.raises(binding.W4A16Error):
        binding.w4a16_quantize(np.zeros((1, 40), np.float32))


# ------------------------------------------------------------------ gemm argument errors

def _call(lib, X, Q, S, Y, M, N, K, group=32, path=None):
    if path is None:
        return lib.w4a16_gemm(X, Q, S, Y, M, N, K, group, None)
    return lib.w4a16_gemm_path(X, Q, S, Y, M, N, K, group, path, None)


BASE = 1 << 40  # fake device addresses; validation never dereferences them
X_, Q_, S_, Y_ = BASE, BASE + (1 << 32), BASE + (2 << 32), BASE + (3 << 32)


def test_gemm_rejects_bad_arguments_synchronously(lib):
    assert _call(lib, X_, Q_, S_, Y_, 1, 8, 64, group=16) == ARG
    assert _call(lib, X_, Q_, S_, Y_, 1, 8, 0) == ARG
    assert _call(lib, X_, Q_, S_, Y_, -1, 8, 64) == ARG
    assert _call(lib, X_, Q_, S_, Y_, 1, -8, 64) == ARG
    assert _call(lib, X_, Q_, S_, Y_, 1, 8, 48) == SHAPE
    assert _call(lib, X_, Q_, S_, Y_, 1, 8, 100) == SHAPE
    assert _call(lib, X_, Q_, S_, Y_, 1, 8, (1 << 17) + 32) == SHAPE
    # the largest K passes validation (M = 0: nothing is launched)
    assert _call(lib, None, None, None, None, 0, 8, 1 << 17) == OK
    assert _call(lib, None, None, None, None, 0, 8, (1 << 17) + 32) == SHAPE
    assert _call(lib, X_, Q_, S_, Y_, 1 << 31, 8, 64) == SHAPE
    assert _call(lib, None, Q_, S_, Y_, 1, 8, 64) == ARG
    assert _call(lib, X_, None, S_, Y_, 1, 8, 64) == ARG
    assert _call(lib, X_, Q_, None, Y_, 1, 8, 64) == ARG
    assert _call(lib, X_, Q_, S_, None, 1, 8, 64) == ARG
    assert _call(lib, X_ + 4, Q_, S_, Y_, 1, 8, 64) == ALIGN
    assert _call(lib, X_, Q_ + 8, S_, Y_, 1, 8, 64) == ALIGN
    assert _call(lib, X_, Q_, S_ + 2, Y_, 1, 8, 64) == ALIGN
    assert _call(lib, X_, Q_, S_, Y_ + 1, 1, 8, 64) == ALIGN
    assert _call(lib, X_, Q_, S_, X_ + 64, 1, 8, 64) == ARG        # Y overlaps X
    assert _call(lib, X_, Q_, S_, Q_ + 16, 1, 8, 64) == ARG        # Y overlaps qweight
    assert _call(lib, X_, Q_, S_, S_, 1, 8, 64) == ARG             # Y overlaps scales
    assert _call(lib, X_, Q_, S_, Y_, 1, 8, 64, path=3) == ARG
    assert _call(lib, X_, Q_, S_, Y_, 1, 8, 64, path=-1) == ARG


def test_gemm_empty_is_a_noop(lib):
    # M == 0 or N == 0: OK without touching the GPU (no device exists here)
    assert _call(lib, None, None, None, None, 0, 8, 64) == OK
    assert _call(lib, None, None, None, None, 3, 0, 64) == OK
    assert _call(lib, None, None, None, None, 0, 0, 32, path=2) == OK
    # ...but K is still validated
    assert _call(lib, None, None, None, None, 0, 8, 40) == SHAPE


W_ = BASE + (4 << 32)  # fake workspace


def _split(lib, X, Q, S, Y, M, N, K, ws=W_, ws_bytes=None, group=32):
    if ws_bytes is None:
        ws_bytes = lib.w4a16_split_workspace_bytes(M, N, K)
    return lib.w4a16_gemm_split(X, Q, S, Y, M, N, K, group, ws, ws_bytes, None)


def test_split_workspace_size(lib):
    ws = lib.w4a16_split_workspace_bytes
    assert ws(0, 8, 64) == 0 and ws(1, 0, 64) == 0 and ws(1, 8, 48) == 0 and ws(1, 8, 0) == 0
    for M, N, K in [(1, 1, 32), (5, 300, 2048), (64, 4096, 7168), (4096, 4096, 7168)]:
        b = ws(M, N, K)
        # at least the two fp16 limbs of every activation plus one exponent per row
        assert b >= 4 * M * K + 4 * M and b % 256 == 0
    assert ws(128, 4096, 7168) >= ws(64, 4096, 7168)


def test_split_rejects_bad_workspace(lib):
    M, N, K = 3, 40, 256
    need = lib.w4a16_split_workspace_bytes(M, N, K)
    assert _split(lib, X_, Q_, S_, Y_, M, N, K, ws=None) == ARG
    assert _split(lib, X_, Q_, S_, Y_, M, N, K, ws=W_ + 128) == ARG      # not 256-aligned
    assert _split(lib, X_, Q_, S_, Y_, M, N, K, ws_bytes=need - 1) == ARG
    assert _split(lib, X_, Q_, S_, Y_, M, N, K, ws=X_) == ARG            # overlaps X
    assert _split(lib, X_, Q_, S_, Y_, M, N, K, ws=Y_ - 256) == ARG      # overlaps Y
    assert _split(lib, X_, Q_, S_, Y_, M, N, K, ws=Q_) == ARG            # overlaps qweight
    assert _split(lib, X_, Q_, S_, Y_, M, N, K, ws=S_) == ARG            # overlaps scales
    # operand errors are those of w4a16_gemm
    assert _split(lib, X_, Q_, S_, Y_, M, N, 48) == SHAPE
    assert _split(lib, X_ + 4, Q_, S_, Y_, M, N, K) == ALIGN
    assert _split(lib, X_, Q_, S_, Y_, M, N, K, group=64) == ARG
    # empty: no workspace needed, nothing launched
    assert _split(lib, None, None, None, None, 0, N, K, ws=None, ws_bytes=0) == OK


def test_split_pack_size_and_errors(lib):
    pb = lib.w4a16_split_pack_bytes
    assert pb(0, 64) == 0 and pb(8, 48) == 0 and pb(8, 0) == 0
    assert pb(1, 32) == 2560 and pb(64, 64) == 2560 and pb(65, 96) == 2 * 2 * 2560
    assert pb(4096, 7168) == 64 * 112 * 2560
    P_ = BASE + (5 << 32)
    need = pb(70, 224)
    pack = lambda q, s, n, k, p, nb, group=32: lib.w4a16_split_pack(q, s, n, k, group, p, nb, None)
    assert pack(Q_, S_, 70, 224, P_, need - 1) == ARG
    assert pack(Q_, S_, 70, 224, None, need) == ARG
    assert pack(Q_, S_, 70, 224, P_ + 8, need) == ARG   # packed not 16-byte aligned
    assert pack(Q_ + 4, S_, 70, 224, P_, need) == ALIGN
    assert pack(Q_, S_, 70, 224, Q_, need) == ARG       # overlaps qweight
    assert pack(Q_, S_, 70, 48, P_, need) == SHAPE
    assert pack(Q_, S_, 70, 224, P_, need, group=64) == ARG
    assert pack(None, None, 0, 224, None, 0) == OK      # N == 0: nothing to do


def test_split_packed_gemm_errors(lib):
    P_ = BASE + (5 << 32)
    M, N, K = 3, 40, 256
    need = lib.w4a16_split_workspace_bytes(M, N, K)
    g = lambda x, p, y, ws=W_, nb=need, m=M, k=K, group=32: lib.w4a16_gemm_split_packed(
        x, p, y, m, N, k, group, ws, nb, None)
    assert g(X_, P_, Y_, ws=None) == ARG
    assert g(X_, P_, Y_, nb=need - 1) == ARG
    assert g(X_, P_, Y_, ws=W_ + 64) == ARG
    assert g(X_, P_ + 4, Y_) == ALIGN
    assert g(X_ + 4, P_, Y_) == ALIGN
    assert g(X_, P_, X_ + 64) == ARG                    # Y overlaps X
    assert g(X_, P_, P_) == ARG                         # Y overlaps packed
    assert g(X_, P_, Y_, k=48) == SHAPE
    assert g(X_, P_, Y_, group=16) == ARG
    assert g(None, None, None, ws=None, nb=0, m=0) == OK


def test_swiglu_rejects_bad_arguments(lib):
    sw = lambda x, q, s_, y, m, f, k, group=32: lib.w4a16_gemm_swiglu(x, q, s_, y, m, f, k, group, None)
    assert sw(X_, Q_, S_, Y_, 1, 8, 48) == SHAPE
    assert sw(X_, Q_, S_, Y_, 1, -1, 64) == ARG
    assert sw(X_, Q_, S_, Y_, 1, 8, 64, group=16) == ARG
    assert sw(None, Q_, S_, Y_, 1, 8, 64) == ARG
    assert sw(X_ + 4, Q_, S_, Y_, 1, 8, 64) == ALIGN
    assert sw(X_, Q_, S_, X_ + 64, 1, 8, 64) == ARG      # Y overlaps X
    assert sw(X_, Q_, S_, Y_, 1, 1 << 30, 64) == SHAPE   # 2F above the row limit
    assert sw(None, None, None, None, 0, 8, 64) == OK
    assert sw(None, None, None, None, 3, 0, 64) == OK


def test_grouped_rejects_bad_arguments(lib):
    I_, O_ = BASE + (6 << 32), BASE + (7 << 32)  # fake token_index, expert_offsets
    gr = lambda x, ti, off, q, s_, y, T, R, E, N, K, group=32: lib.w4a16_gemm_grouped(
        x, ti, off, q, s_, y, T, R, E, N, K, group, None)
    assert gr(X_, I_, O_, Q_, S_, Y_, 4, 8, 3, 16, 48) == SHAPE
    assert gr(X_, I_, O_, Q_, S_, Y_, 4, 8, 0, 16, 64) == ARG        # no experts
    assert gr(X_, I_, O_, Q_, S_, Y_, 4, 8, 70000, 16, 64) == SHAPE  # too many experts
    assert gr(X_, I_, O_, Q_, S_, Y_, 0, 8, 3, 16, 64) == ARG        # slots, no tokens
    assert gr(X_, I_, O_, Q_, S_, Y_, 4, -1, 3, 16, 64) == ARG
    assert gr(X_, None, O_, Q_, S_, Y_, 4, 8, 3, 16, 64) == ARG
    assert gr(X_, I_, None, Q_, S_, Y_, 4, 8, 3, 16, 64) == ARG
    assert gr(X_ + 4, I_, O_, Q_, S_, Y_, 4, 8, 3, 16, 64) == ALIGN
    assert gr(X_, I_ + 2, O_, Q_, S_, Y_, 4, 8, 3, 16, 64) == ALIGN
    assert gr(X_, I_, O_, Q_, S_, X_ + 64, 4, 8, 3, 16, 64) == ARG   # Y overlaps X
    assert gr(X_, I_, O_, Q_, S_, I_, 4, 8, 3, 16, 64) == ARG         # Y overlaps token_index
    assert gr(X_, I_, O_, Q_, S_, Y_, 4, 8, 3, 16, 64, group=16) == ARG
    assert gr(None, None, None, None, None, None, 0, 0, 3, 16, 64) == OK   # no slots
    assert gr(None, None, None, None, None, None, 4, 8, 3, 0, 64) == OK    # N == 0


def test_binding_refuses_host_tensors(lib):
    torch = pytest.importorskip("torch")
    X = torch.zeros(1, 64)
    with pytest.raises(TypeError):
        binding.w4a16_gemm(X, torch.zeros(8, 8, dtype=torch.int32), torch.zeros(8, 2))


def test_header_names_match_binding():
    assert set(binding.header_functions()) == set(binding._SIGS)
    assert isinstance(ctypes.sizeof(ctypes.c_void_p), int)


def test_grouped_kernel_choice():
    """w4a16_grouped_kernel: the matrix-core kernel for decode-shaped MoE, the
    FMA kernels past its limits, 0 for refused shapes (host only)."""
    from int4_weight_only_03_amd import binding as b
    assert b.w4a16_grouped_kernel(16, 64, 32, 1024, 7168) == b.W4A16_GROUPED_MFMA
    assert b.w4a16_grouped_kernel(1, 8, 256, 2048, 7168) == b.W4A16_GROUPED_MFMA
    assert b.w4a16_grouped_kernel(6, 18, 4100, 20, 96) == b.W4A16_GROUPED_ROWS
    assert b.w4a16_grouped_kernel(3, 3, 2, 8, 40992) == b.W4A16_GROUPED_GEMV
    for bad in [(0, 1, 1, 8, 32), (1, 1, 0, 8, 32), (1, 1, 1, 8, 48), (1, 1, 65536, 8, 32),
                (1, 0, 1, 8, 32)]:
        assert b.w4a16_grouped_kernel(*bad) == 0


def test_grouped_pack_size_and_errors(lib):
    pb = lib.w4a16_grouped_pack_bytes
    assert pb(0, 16, 128) == 0 and pb(1, 16, 48) == 0 and pb(1, 0, 128) == 0
    assert pb(1, 16, 128) == 1280 and pb(1, 17, 160) == 2 * 2 * 1280
    assert pb(32, 1024, 7168) == 32 * 64 * 56 * 1280
    P_ = BASE + (5 << 32)
    need = pb(3, 40, 224)
    pack = lambda q, s, e, n, k, p, nb, group=32: lib.w4a16_grouped_pack(q, s, e, n, k, group, p,
                                                                         nb, None)
    assert pack(Q_, S_, 3, 40, 224, P_, need - 1) == ARG
    assert pack(Q_, S_, 3, 40, 224, None, need) == ARG
    assert pack(Q_, S_, 3, 40, 224, P_ + 8, need) == ARG   # packed not 16-byte aligned
    assert pack(Q_ + 4, S_, 3, 40, 224, P_, need) == ALIGN
    assert pack(Q_, S_, 3, 40, 224, Q_, need) == ARG       # overlaps qweight
    assert pack(Q_, S_, 3, 40, 48, P_, need) == SHAPE
    assert pack(Q_, S_, 0, 40, 224, P_, need) == ARG
    assert pack(Q_, S_, 65536, 40, 224, P_, need) == SHAPE
    assert pack(Q_, S_, 3, 40, 224, P_, need, group=64) == ARG
    assert pack(None, None, 3, 0, 224, None, 0) == OK      # N == 0: nothing to do


def test_grouped_packed_gemm_errors(lib):
    I_, O_, P_ = BASE + (6 << 32), BASE + (7 << 32), BASE + (5 << 32)
    g = lambda x, p, y, t=16, r=64, e=32, n=64, k=256, group=32: lib.w4a16_gemm_grouped_packed(
        x, I_, O_, p, y, t, r, e, n, k, group, None)
    assert g(X_, P_, Y_, e=4100) == SHAPE                 # not a matrix-core shape
    assert g(X_, P_, Y_, k=40992, e=2) == SHAPE           # K too long to stage
    assert g(X_, P_ + 4, Y_) == ALIGN
    assert g(X_ + 4, P_, Y_) == ALIGN
    assert g(None, P_, Y_) == ARG
    assert g(X_, None, Y_) == ARG
    assert g(X_, P_, X_ + 64) == ARG                      # Y overlaps X
    assert g(X_, P_, P_ + 64) == ARG                      # Y overlaps packed
    assert g(X_, P_, Y_, k=48) == SHAPE
    assert g(X_, P_, Y_, group=16) == ARG
    assert g(X_, P_, Y_, t=0) == ARG                      # slots but no tokens
    assert g(None, None, None, r=0) == OK


def test_repack_trio_errors(lib):
    """The repack entry points: sizes, and argument errors before any launch."""
    P_ = BASE + (5 << 32)
    # ceil(N/16) * ceil(K/128) * 1280 bytes: 16-row tiles, 4-group steps of 1 KB
    # of weights and 256 B of scales
    assert lib.w4a16_repacked_bytes(4096, 7168, 32) == 256 * 56 * 1280
    assert lib.w4a16_repacked_bytes(17, 96, 32) == 2 * 1 * 1280
    assert lib.w4a16_repacked_bytes(4096, 7168, 16) == 0
    assert lib.w4a16_repacked_bytes(4096, 48, 32) == 0
    assert lib.w4a16_repacked_bytes(0, 7168, 32) == 0
    assert lib.w4a16_repacked_bytes(64, (1 << 17) + 32, 32) == 0
    r = lambda q, s_, p, n=64, k=256, group=32: lib.w4a16_repack(q, s_, p, n, k, group, None)
    assert r(Q_, S_, P_, k=48) == SHAPE
    assert r(Q_, S_, P_, k=(1 << 17) + 32) == SHAPE
    assert r(Q_, S_, P_, group=16) == ARG
    assert r(Q_, S_, P_, n=-1) == ARG
    assert r(None, S_, P_) == ARG
    assert r(Q_, S_, None) == ARG
    assert r(Q_ + 4, S_, P_) == ALIGN
    assert r(Q_, S_ + 2, P_) == ALIGN
    assert r(Q_, S_, P_ + 4) == ALIGN
    assert r(Q_, S_, Q_ + 64) == ARG                      # packed overlaps qweight
    assert r(Q_, S_, S_ + 64) == ARG                      # packed overlaps scales
    assert r(None, None, None, n=0) == OK
    g = lambda x, p, y, m=1, n=64, k=256, group=32: lib.w4a16_gemm_repacked(
        x, p, y, m, n, k, group, None)
    assert g(X_, P_, Y_, k=48) == SHAPE
    assert g(X_, P_, Y_, k=(1 << 17) + 32) == SHAPE
    assert g(X_, P_ + 4, Y_) == ALIGN
    assert g(X_ + 4, P_, Y_) == ALIGN
    assert g(X_, P_, Y_ + 2) == ALIGN
    assert g(None, P_, Y_) == ARG
    assert g(X_, None, Y_) == ARG
    assert g(X_, P_, X_ + 64) == ARG                      # Y overlaps X
    assert g(X_, P_, P_ + 64) == ARG                      # Y overlaps packed
    assert g(X_, P_, Y_, group=16) == ARG
    assert g(X_, P_, Y_, m=-1) == ARG
    assert g(None, None, None, m=0) == OK
    assert g(None, None, None, n=0) == OK


def test_small_packed_errors(lib):
    P_, W_ = BASE + (5 << 32), BASE + (6 << 32)
    need = lib.w4a16_small_packed_workspace_bytes(64, 4096, 7168)
    # 16 groups of 256 columns x 2 chunks of 32 rows x 8 K slices of 7 steps
    # (896 k): 256 workgroups, 8 partial results
    assert need == 8 * 64 * 4096 * 4
    assert lib.w4a16_small_packed_workspace_bytes(4, 16, 128) == 0    # one slice: no partials
    assert lib.w4a16_small_packed_workspace_bytes(65, 4096, 7168) == 0
    assert lib.w4a16_small_packed_workspace_bytes(8, 4096, 48) == 0
    g = lambda x, p, y, m=64, n=4096, k=7168, group=32, ws=W_, wsb=need: \
        lib.w4a16_gemm_small_packed(x, p, y, m, n, k, group, ws, wsb, None)
    assert g(X_, P_, Y_, m=65) == SHAPE
    assert g(X_, P_, Y_, k=48) == SHAPE
    assert g(X_, P_, Y_, group=16) == ARG
    assert g(X_ + 4, P_, Y_) == ALIGN
    assert g(X_, P_ + 4, Y_) == ALIGN
    assert g(None, P_, Y_) == ARG
    assert g(X_, P_, X_ + 64) == ARG                      # Y overlaps X
    assert g(X_, P_, P_ + 64) == ARG                      # Y overlaps packed
    assert g(X_, P_, Y_, ws=None) == ARG                  # partials need a workspace
    assert g(X_, P_, Y_, ws=W_ + 16) == ARG               # not 256-byte aligned
    assert g(X_, P_, Y_, wsb=need - 4) == ARG             # too small
    assert g(X_, P_, Y_, ws=X_) == ARG                    # overlaps X
    assert g(X_, P_, Y_, ws=Y_) == ARG                    # overlaps Y
    assert g(None, None, None, m=0) == OK
    assert g(None, None, None, n=0) == OK


def test_small_packed_noalloc_errors(lib):
    """Refusals of the allocation-free entry point, all before any GPU work."""
    P_ = BASE + (5 << 32)
    g = lambda x, p, y, m=64, n=4096, k=7168, group=32: \
        lib.w4a16_gemm_small_packed_noalloc(x, p, y, m, n, k, group, None)
    # partials beyond the fixed 64 MiB: 7 K slices x 64 x 65536 floats
    assert lib.w4a16_small_packed_workspace_bytes(64, 65536, 7168) > 64 << 20
    assert lib.w4a16_small_packed_workspace_bytes(64, 32768, 7168) <= 64 << 20
    assert g(X_, P_, Y_, n=65536) == SCRATCH
    assert g(X_, P_, Y_, m=65) == SHAPE
    assert g(X_, P_, Y_, k=48) == SHAPE
    assert g(X_, P_, Y_, group=16) == ARG
    assert g(X_ + 4, P_, Y_) == ALIGN
    assert g(X_, P_ + 4, Y_) == ALIGN
    assert g(None, P_, Y_) == ARG
    assert g(X_, P_, X_ + 64) == ARG                      # Y overlaps X
    assert g(X_, P_, P_ + 64) == ARG                      # Y overlaps packed
    assert g(None, None, None, m=0) == OK
    assert g(None, None, None, n=0) == OK


def test_one_hip_runtime_per_process():
    # loading the library first in a fresh process still maps a single HIP
    # runtime, torch's: a second copy would initialise the GPU a second time
    # and see no device
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from int4_weight_only_03_amd import binding\n"
            "binding.load()\n"
            "import torch, os\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(sorted(maps)); print(os.path.dirname(torch.__file__))\n") % root
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    maps_line, torch_dir = out.stdout.strip().splitlines()[-2:]
    maps = eval(maps_line)
    assert len(maps) == 1, maps
    assert os.path.realpath(maps[0]).startswith(os.path.realpath(torch_dir)), (maps, torch_dir)
