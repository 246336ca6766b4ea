"""Plain, slow, obviously correct CPU oracle of the W4A16 group-quantized GEMM.

Test infrastructure only: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

What is computed, and where the pages state it
----------------------------------------------
Pages are cited by title and section:

* "The Silence of Success: A Single Line That Speaks Volumes", section "What
  the Edit Actually Built": fp32 activations times int4 weights held two
  4-bit values per byte, one scale per group of 32 input columns; the golden
  result is numpy's dequantize-then-multiply.
* "The Quiet Commit: How a Single Documentation Edit Marks the Completion of
  a Major Engineering Milestone", section "The INT4 Milestone": symmetric
  quantization, 8 nibbles per int32 along the input dimension, value =
  nibble - 8, fp32 per-group scales; golden outputs computed from the
  dequantized weights.  Section "Input Knowledge Required" repeats group 32,
  8 nibbles per int32 and value = nibble - 8.
* "The Quiet Commit: How a Single Plan Update Closed Phase 3 of a Native DDTree
  Inference Engine", section "The Context: Phase 3 of a Custom Inference
  Stack": symmetric per-group quantization, group 32, 8 nibbles per int32
  along the input dimension.

Readings taken where the pages are silent (each is listed in the design doc):

* Layout: W is [N][K] (N outputs, K inputs), Y = X . dequant(W)^T.
  ``qweight[n][j]`` holds k = 8j + i in bits 4i..4i+3, i = 0..7, low nibble
  first; on a little-endian machine byte b of the word then holds k = 8j+2b
  (low half) and 8j+2b+1 (high half), which is the "two 4-bit values per
  byte" the first page describes.  Unpacking uses logical shifts on the
  unsigned word (a word whose nibble 7 is >= 8 is negative as int32).
* Scale: scale = max|w| / 7 over the group, one fp32 true division rounded
  to nearest even.
* Code: q = clamp(rint(w / scale), -8, 7) with an fp32 true division and
  round-half-to-even; nibble = q + 8.  A group whose scale is 0 (all zero,
  or so tiny that max|w|/7 underflows) gets q = 0 everywhere.
* Non-finite weights are rejected; K % 32 != 0 is rejected (no padding).
* Dequantized weight = fl32((nibble - 8) * scale), one rounded fp32 multiply.
* Repack: the pages describe no repack step; the library adds an optional
  one-time repack of the weights into layouts private to its kernels.
  ``pack_split`` writes the split-path layout from its index formula (64-row
  slabs, stages of 2 groups, zero code and zero scale as padding) and
  ``pack_grouped`` the grouped one; they only move bits, so the library's
  repacks must match them byte for byte.
* Grouped (MoE) GEMM: routed slot r of expert e is the product of token
  token_index[r] with expert e's weights (the pages run the MoE experts
  through the INT4 path); ``grouped_gemm`` applies ``gemm`` expert by expert
  to the gathered token rows, and the tolerance is that of ``gemm``.
* Fused gate/up SwiGLU (the pages' decode configuration is the gate+up matrix,
  2 x 2048 rows; SwiGLU is the engine's MLP activation): W holds the gate rows
  then the up rows; the result is silu(g) * u with silu(v) = v / (1 + e^-v),
  evaluated in fp64 from the fp64 products.  Acceptance propagates the GEMM
  bound of g and u through silu (|silu'| <= 1.1) and adds the rounding of an
  fp32 evaluation of the epilogue (``compare_swiglu``).
* Product: accumulated in fp64 (every fp32 x fp32 product is exact in fp64).
  An fp32 result is accepted iff |Y - Y_ref| <= 1e-5 * sum_k |x_k w_k| + 1e-6
  elementwise, with w the dequantized fp32 weight and the sum in fp64.
"""

from __future__ import annotations

import numpy as np

GROUP = 32
REL_TOL = 1e-5
ABS_TOL = 1e-6

_F32 = np.float32


def check_k(K: int) -> None:
    """K must be a positive multiple of the group width (no padding path)."""
    if K <= 0 or K % GROUP != 0:
        raise ValueError(f"K={K} is not a positive multiple of {GROUP}")


# --------------------------------------------------------------------------
# quantize: "symmetric per-group quantization, group size 32"
# --------------------------------------------------------------------------

def quantize(W: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """W fp32 [N][K] -> (qweight int32 [N][K/8], scales fp32 [N][K/32]).

    Steps, in order: group the K axis in runs of 32; scale = max|w| / 7 (fp32);
    q = rint(w / scale) (fp32 division, ties to even), clamped to [-8, 7];
    nibble = q + 8; pack 8 nibbles per word, low nibble first.
    """
    W = np.asarray(W)
    if W.dtype != np.float32 or W.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    N, K = W.shape
    check_k(K)
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    G = K // GROUP
    Wg = W.reshape(N, G, GROUP)
    amax = np.max(np.abs(Wg), axis=2)                 # exact
    scale = (amax / _F32(7.0)).astype(np.float32)     # fp32 true division
    zero = scale == 0
    safe = np.where(zero, _F32(1.0), scale).astype(np.float32)
    ratio = (Wg / safe[:, :, None]).astype(np.float32)  # fp32 true division
    q = np.rint(ratio)                                 # round half to even
    q = np.where(zero[:, :, None], _F32(0.0), q)
    q = np.clip(q, -8, 7)
    nib = (q.astype(np.int64) + 8).astype(np.uint8).reshape(N, K)
    return pack(nib), scale


# --------------------------------------------------------------------------
# pack / unpack: "8 nibbles per int32 along the input dimension"
# --------------------------------------------------------------------------

def pack(nib: np.ndarray) -> np.ndarray:
    """nibbles [N][K] (values 0..15) -> int32 [N][K/8], nibble i of word j = k 8j+i."""
    nib = np.asarray(nib)
    N, K = nib.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8 to pack")
    if np.any((nib.astype(np.int64) < 0) | (nib.astype(np.int64) > 15)):
        raise ValueError("nibble out of range")
    words = np.zeros((N, K // 8), dtype=np.uint64)
    for i in range(8):
        words |= nib[:, i::8].astype(np.uint64) << np.uint64(4 * i)
    return words.astype(np.uint32).view(np.int32)


def unpack(qweight: np.ndarray) -> np.ndarray:
    """int32 [N][K/8] -> nibbles uint8 [N][K] (logical shifts on the unsigned word)."""
    u = np.asarray(qweight, dtype=np.int32).view(np.uint32)
    N, J = u.shape
    nib = np.empty((N, 8 * J), dtype=np.uint8)
    for i in range(8):
        nib[:, i::8] = ((u >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.uint8)
    return nib


# --------------------------------------------------------------------------
# dequantize: "value = nibble - 8", times the group's fp32 scale
# --------------------------------------------------------------------------

def dequantize(qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp32 [N][K] with w = fl32((nibble - 8) * scale[n][k // 32])."""
    nib = unpack(qweight)
    N, K = nib.shape
    scales = np.asarray(scales, dtype=np.float32)
    if scales.shape != (N, K // GROUP):
        raise ValueError(f"scales shape {scales.shape} != {(N, K // GROUP)}")
    centred = nib.astype(np.float32) - _F32(8.0)             # exact small integers
    s = np.repeat(scales, GROUP, axis=1)                       # scale of k's group
    return (centred * s).astype(np.float32)                    # one fp32 multiply


# --------------------------------------------------------------------------
# the product, accumulated in fp64 ("dequantize-then-multiply")
# --------------------------------------------------------------------------

SLAB = 64          # rows per slab of the split-path packed layout
STAGE_GROUPS = 2   # groups per stage


def pack_split(qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed split-path layout of (qweight[N][K/8], scales[N][K/32]) as bytes.

    For slab s (rows 64s..64s+63) and stage t (groups 2t, 2t+1), with S slabs
    and T stages: 16-byte chunk ((s*T + t)*2 + g)*64 + r holds the 4 words of
    group 2t+g of row 64s+r; after all S*T*2048 such bytes, float
    (s*T + t)*128 + 2r + g holds that group's scale.  Rows past N and the group
    past G = K/32 (odd G) hold words 0x88888888 (every nibble 8, code 0) and
    scale 0.0.
    """
    qweight = np.ascontiguousarray(qweight).view(np.uint32)
    scales = np.ascontiguousarray(scales, dtype=_F32)
    N, G = scales.shape
    if qweight.shape != (N, 4 * G):
        raise ValueError("qweight and scales disagree")
    S = -(-N // SLAB)
    T = -(-G // STAGE_GROUPS)
    words = np.full((S, T, STAGE_GROUPS, SLAB, 4), 0x88888888, dtype=np.uint32)
    sc = np.zeros((S, T, SLAB, STAGE_GROUPS), dtype=_F32)
    for n in range(N):                      # plain loops: row n, group gg
        s_, r = divmod(n, SLAB)
        for gg in range(G):
            t, g = divmod(gg, STAGE_GROUPS)
            words[s_, t, g, r, :] = qweight[n, 4 * gg:4 * gg + 4]
            sc[s_, t, r, g] = scales[n, gg]
    return np.concatenate([words.reshape(-1).view(np.uint8), sc.reshape(-1).view(np.uint8)])


def unpack_split(packed: np.ndarray, N: int, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Inverse of pack_split: (qweight int32 [N][K/8], scales fp32 [N][K/32])."""
    check_k(K)
    G = K // GROUP
    S = -(-N // SLAB)
    T = -(-G // STAGE_GROUPS)
    nw = S * T * STAGE_GROUPS * SLAB * 4
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    words = packed[:4 * nw].view(np.uint32).reshape(S, T, STAGE_GROUPS, SLAB, 4)
    sc = packed[4 * nw:4 * nw + 4 * S * T * SLAB * STAGE_GROUPS].view(_F32).reshape(
        S, T, SLAB, STAGE_GROUPS)
    qweight = np.zeros((N, 4 * G), dtype=np.uint32)
    scales = np.zeros((N, G), dtype=_F32)
    for n in range(N):
        s_, r = divmod(n, SLAB)
        for gg in range(G):
            t, g = divmod(gg, STAGE_GROUPS)
            qweight[n, 4 * gg:4 * gg + 4] = words[s_, t, g, r, :]
            scales[n, gg] = sc[s_, t, r, g]
    return qweight.view(np.int32), scales


TILE_ROWS = 16     # grouped repack: weight rows per tile
STEP_GROUPS = 4    # grouped repack: groups per step


def pack_grouped(qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed grouped-path layout of (qweight[E][N][K/8], scales[E][N][K/32])
    as bytes.

    For expert e, tile t (rows 16t..16t+15) and step s (groups 4s..4s+3),
    with T16 tiles and S4 steps, block b = (e*T16 + t)*S4 + s: 16-byte chunk
    b*64 + c + 16R holds word R of groups 4s..4s+3 (in that order) of row
    16t + c; after all E*T16*S4*1024 such bytes, float (b*16 + c)*4 + q holds
    the scale of group 4s + q of row 16t + c.  Rows past N and groups past G
    hold words 0x88888888 (every nibble 8, code 0) and scale 0.0.
    """
    qweight = np.ascontiguousarray(qweight).view(np.uint32)
    scales = np.ascontiguousarray(scales, dtype=_F32)
    E, N, G = scales.shape
    if qweight.shape != (E, N, 4 * G):
        raise ValueError("qweight and scales disagree")
    T16 = -(-N // TILE_ROWS)
    S4 = -(-G // STEP_GROUPS)
    words = np.full((E, T16, S4, 4, TILE_ROWS, STEP_GROUPS), 0x88888888, dtype=np.uint32)
    sc = np.zeros((E, T16, S4, TILE_ROWS, STEP_GROUPS), dtype=_F32)
    for e in range(E):                      # plain loops: expert, row, group, word
        for n in range(N):
            t, c = divmod(n, TILE_ROWS)
            for g in range(G):
                s_, q = divmod(g, STEP_GROUPS)
                for R in range(4):
                    words[e, t, s_, R, c, q] = qweight[e, n, 4 * g + R]
                sc[e, t, s_, c, q] = scales[e, n, g]
    return np.concatenate([words.reshape(-1).view(np.uint8), sc.reshape(-1).view(np.uint8)])


def unpack_grouped(packed: np.ndarray, E: int, N: int, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Inverse of pack_grouped: (qweight int32 [E][N][K/8], scales fp32 [E][N][K/32])."""
    check_k(K)
    G = K // GROUP
    T16 = -(-N // TILE_ROWS)
    S4 = -(-G // STEP_GROUPS)
    nw = E * T16 * S4 * 4 * TILE_ROWS * STEP_GROUPS
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    words = packed[:4 * nw].view(np.uint32).reshape(E, T16, S4, 4, TILE_ROWS, STEP_GROUPS)
    sc = packed[4 * nw:4 * nw + 4 * E * T16 * S4 * TILE_ROWS * STEP_GROUPS].view(_F32).reshape(
        E, T16, S4, TILE_ROWS, STEP_GROUPS)
    qweight = np.zeros((E, N, 4 * G), dtype=np.uint32)
    scales = np.zeros((E, N, G), dtype=_F32)
    for e in range(E):
        for n in range(N):
            t, c = divmod(n, TILE_ROWS)
            for g in range(G):
                s_, q = divmod(g, STEP_GROUPS)
                for R in range(4):
                    qweight[e, n, 4 * g + R] = words[e, t, s_, R, c, q]
                scales[e, n, g] = sc[e, t, s_, c, q]
    return qweight.view(np.int32), scales


def _operands(X, qweight, scales):
    X = np.asarray(X)
    if X.dtype != np.float32 or X.ndim != 2:
        raise TypeError("X must be a 2-D float32 array")
    check_k(X.shape[1])
    Wd = dequantize(qweight, scales)
    if Wd.shape[1] != X.shape[1]:
        raise ValueError("K of X and of the weights differ")
    return X, Wd


def gemm(X: np.ndarray, qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Y_ref[M][N] = X . dequant(W)^T, every product and sum in fp64."""
    X, Wd = _operands(X, qweight, scales)
    return X.astype(np.float64) @ Wd.astype(np.float64).T


def abs_gemm(X: np.ndarray, qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """T[M][N] = sum_k |x_k| |w_k| in fp64 (the scale of the tolerance)."""
    X, Wd = _operands(X, qweight, scales)
    return np.abs(X).astype(np.float64) @ np.abs(Wd).astype(np.float64).T


def gemm_entries(X, qweight, scales, rows, cols):
    """(Y_ref, T) at the listed (row, col) pairs only, one dot product each.

    For full-size problems where the whole fp64 product would be slow: each
    entry dequantizes one weight row and takes one fp64 dot product.
    """
    X = np.asarray(X)
    check_k(X.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    y = np.empty(rows.shape, dtype=np.float64)
    t = np.empty(rows.shape, dtype=np.float64)
    cache = {}
    for idx, (m, n) in enumerate(zip(rows.tolist(), cols.tolist())):
        if n not in cache:
            cache[n] = dequantize(qweight[n:n + 1], scales[n:n + 1])[0].astype(np.float64)
        w = cache[n]
        x = X[m].astype(np.float64)
        y[idx] = float(np.dot(x, w))
        t[idx] = float(np.dot(np.abs(x), np.abs(w)))
    return y, t


# --------------------------------------------------------------------------
# acceptance
# --------------------------------------------------------------------------

def bound(T: np.ndarray) -> np.ndarray:
    """Allowed |Y - Y_ref|: 1e-5 * sum_k |x_k w_k| + 1e-6."""
    return REL_TOL * np.asarray(T, dtype=np.float64) + ABS_TOL


def _verdict(Y, Yref, T) -> dict:
    Y = np.asarray(Y, dtype=np.float64)
    err = np.abs(Y - Yref)
    ratio = err / bound(T)
    finite = bool(np.all(np.isfinite(Y)))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return {
        "ok": finite and worst <= 1.0,
        "max_ratio": worst,
        "max_abs_err": float(np.max(err)) if err.size else 0.0,
        "finite": finite,
        "n": int(ratio.size),
    }


def compare_to(Y: np.ndarray, Yref: np.ndarray, T: np.ndarray) -> dict:
    """The acceptance verdict of Y against a Y_ref = gemm(...) and T = abs_gemm(...)
    computed once (for large problems checked on several paths)."""
    if np.shape(Y) != np.shape(Yref):
        raise ValueError(f"Y shape {np.shape(Y)} != {np.shape(Yref)}")
    return _verdict(Y, Yref, T)


def compare(Y: np.ndarray, X: np.ndarray, qweight: np.ndarray, scales: np.ndarray) -> dict:
    """Check every element of an fp32 result against the fp64 oracle."""
    Yref = gemm(X, qweight, scales)
    T = abs_gemm(X, qweight, scales)
    if np.shape(Y) != Yref.shape:
        raise ValueError(f"Y shape {np.shape(Y)} != {Yref.shape}")
    return _verdict(Y, Yref, T)


def check_routing(token_index: np.ndarray, offsets: np.ndarray, T: int, E: int) -> None:
    """Routing must be well formed: offsets non-decreasing from 0 to R, token
    indices in [0, T)."""
    token_index = np.asarray(token_index)
    offsets = np.asarray(offsets)
    R = token_index.size
    if offsets.shape != (E + 1,) or offsets[0] != 0 or offsets[-1] != R:
        raise ValueError("expert offsets must run from 0 to R with E + 1 entries")
    if np.any(np.diff(offsets) < 0):
        raise ValueError("expert offsets must be non-decreasing")
    if R and (token_index.min() < 0 or token_index.max() >= T):
        raise ValueError("token index out of range")


def grouped_gemm(X, token_index, offsets, qweight, scales) -> np.ndarray:
    """Y[r] = X[token_index[r]] . dequant(W_e)^T for the expert e owning slot r (fp64)."""
    E, N = qweight.shape[0], qweight.shape[1]
    check_routing(token_index, offsets, X.shape[0], E)
    Y = np.zeros((len(token_index), N))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            Y[r0:r1] = gemm(X[token_index[r0:r1]], qweight[e], scales[e])
    return Y


def compare_grouped(Y, X, token_index, offsets, qweight, scales) -> dict:
    """Elementwise check of a grouped result: each expert's rows against gemm."""
    ref = grouped_gemm(X, token_index, offsets, qweight, scales)
    Y = np.asarray(Y, dtype=np.float64)
    T = np.zeros_like(ref)
    for e in range(qweight.shape[0]):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            T[r0:r1] = abs_gemm(X[token_index[r0:r1]], qweight[e], scales[e])
    return _verdict(Y, ref, T)


def silu(v: np.ndarray) -> np.ndarray:
    """silu(v) = v / (1 + exp(-v)) in fp64 (exp overflow for very negative v gives -0)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu(X: np.ndarray, qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """silu(X . gate^T) * (X . up^T) in fp64; W rows 0..F-1 gate, F..2F-1 up."""
    Y = gemm(X, qweight, scales)
    F = Y.shape[1] // 2
    return silu(Y[:, :F]) * Y[:, F:]


SILU_LIPSCHITZ = 1.1   # max |silu'(v)| = 1.0998...
EPILOGUE_ULPS = 8      # fp32 exp, add, divide and multiply, rounded


def swiglu_bound(X: np.ndarray, qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Allowed |Y - swiglu| per output: the GEMM bound e_g, e_u of the gate and
    up sums carried through silu(g) * u, plus the epilogue's fp32 rounding."""
    Y = gemm(X, qweight, scales)
    T = abs_gemm(X, qweight, scales)
    F = Y.shape[1] // 2
    g, u = Y[:, :F], Y[:, F:]
    eg, eu = bound(T[:, :F]), bound(T[:, F:])
    sg = np.abs(silu(g))
    carried = SILU_LIPSCHITZ * eg * (np.abs(u) + eu) + sg * eu
    rounding = EPILOGUE_ULPS * 2.0 ** -24 * (sg + SILU_LIPSCHITZ * eg) * (np.abs(u) + eu)
    return carried + rounding


def compare_swiglu(Y: np.ndarray, X: np.ndarray, qweight: np.ndarray, scales: np.ndarray) -> dict:
    """Elementwise check of a fused gate/up SwiGLU result against swiglu()."""
    ref = swiglu(X, qweight, scales)
    Y = np.asarray(Y, dtype=np.float64)
    if Y.shape != ref.shape:
        raise ValueError(f"shape {Y.shape} != {ref.shape}")
    b = swiglu_bound(X, qweight, scales)
    finite = bool(np.all(np.isfinite(Y)))
    err = np.abs(Y - ref)
    ratio = float(np.max(err / b)) if err.size else 0.0
    return {"ok": finite and bool(np.all(err <= b)), "max_ratio": ratio,
            "max_abs_err": float(err.max()) if err.size else 0.0, "finite": finite,
            "n": int(err.size)}


def compare_entries(Y: np.ndarray, X, qweight, scales, rows, cols) -> dict:
    """Check sampled entries Y[rows[i], cols[i]] against the oracle."""
    Yref, T = gemm_entries(X, qweight, scales, rows, cols)
    got = np.asarray(Y)[np.asarray(rows), np.asarray(cols)]
    return _verdict(got, Yref, T)
