"""Seeded synthetic inputs for the W4A16 group-quantized GEMM.

This module only draws random numbers.  It holds none of the method's
arithmetic (no quantization, packing, dequantization or matrix product), so
both the CPU oracle and the HIP path may take their inputs from it without
sharing any code of the method.

Every array is drawn with ``numpy.random.default_rng(seed)`` in float64 and
cast to float32 last.  Draw order is fixed: X first, then W, then any mask.

The workload shapes stand in for the layers the pages run through the INT4
path (MoE experts, shared expert and dense MLP of a DeepSeek-V3/Kimi-style
model: "The Quiet Commit ... Documentation Edit", section "The INT4
Milestone").  The pages measure no public benchmark or dataset; these
synthetic draws replace the tiny model bundles and real weights they used.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

GROUP = 32  # group width along K (format constant of the weights)


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    seed: int
    x_kind: str  # "gauss", "half_gauss" or "correlated"
    w_kind: str  # "gauss" or "outlier"
    note: str

    @property
    def groups(self) -> int:
        return self.K // GROUP

    def algorithmic_bytes(self) -> int:
        """Bytes the GEMM must move once: packed weights, scales, X and Y."""
        M, N, K = self.M, self.N, self.K
        return N * K // 2 + 4 * N * (K // GROUP) + 4 * M * K + 4 * M * N

    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 512, 0, "gauss", "gauss",
                     "tiny check, fits in cache"),
    "decode_gate_up": Workload("decode_gate_up", 1, 7168, 4096, 1, "gauss", "gauss",
                               "decode GEMV, MoE gate+up projection (2x2048)"),
    "decode_down": Workload("decode_down", 1, 2048, 7168, 2, "half_gauss", "outlier",
                            "decode GEMV, MoE down projection, 1% x10 weight outliers"),
    "verify_tree": Workload("verify_tree", 64, 7168, 4096, 3, "correlated", "gauss",
                            "draft-tree verify batch of 64 correlated tokens"),
    "prefill": Workload("prefill", 4096, 7168, 4096, 4, "gauss", "gauss",
                        "prefill-shaped GEMM"),
}

ORDER = ["tiny", "decode_gate_up", "decode_down", "verify_tree", "prefill"]


@dataclass(frozen=True)
class MoeWorkload:
    """Grouped (MoE) GEMM: T tokens, each routed to `topk` of E experts with
    uniform random routing; every expert has its own N x K weights."""
    name: str
    T: int
    E: int
    topk: int
    N: int
    K: int
    seed: int
    note: str

    @property
    def R(self) -> int:
        return self.T * self.topk

    def algorithmic_bytes(self, offsets: np.ndarray) -> int:
        """Weights and scales of every expert with at least one slot, the token
        rows and the output rows, each moved once."""
        active = int(np.count_nonzero(np.diff(offsets)))
        N, K = self.N, self.K
        return active * (N * K // 2 + 4 * N * (K // GROUP)) + 4 * self.T * K + 4 * self.R * N

    def flops(self) -> int:
        return 2 * self.R * self.N * self.K


MOE_WORKLOADS = {
    "moe_decode": MoeWorkload("moe_decode", 16, 32, 4, 1024, 7168, 5,
                              "decode batch of 16 tokens, top-4 of 32 experts (some empty), "
                              "N=1024 per expert"),
}


def moe_routing(rng: np.random.Generator, T: int, E: int, topk: int):
    """Uniform top-k routing: each token draws topk distinct experts.  Returns
    (token_index int32 [T*topk], expert_offsets int32 [E+1]): slots sorted by
    expert (then token), expert e owning slots offsets[e]..offsets[e+1]-1."""
    choice = np.stack([rng.permutation(E)[:topk] for _ in range(T)])   # [T][topk]
    expert = choice.reshape(-1)
    token = np.repeat(np.arange(T), topk)
    order = np.lexsort((token, expert))
    counts = np.bincount(expert, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return token[order].astype(np.int32), offsets.astype(np.int32)


def moe_case(T: int, E: int, topk: int, N: int, K: int, seed: int):
    """(X [T][K], W [E][N][K], token_index [R], expert_offsets [E+1]).
    Draw order: X, then each expert's W in turn, then the routing."""
    rng = np.random.default_rng(seed)
    X = _draw_x(rng, "gauss", T, K)
    W = np.empty((E, N, K), dtype=np.float32)
    for e in range(E):
        W[e] = _draw_w(rng, "gauss", N, K)
    token_index, offsets = moe_routing(rng, T, E, topk)
    return X, W, token_index, offsets


def make_moe(name: str):
    wl = MOE_WORKLOADS[name]
    return moe_case(wl.T, wl.E, wl.topk, wl.N, wl.K, wl.seed)


def _draw_x(rng: np.random.Generator, kind: str, M: int, K: int) -> np.ndarray:
    if kind == "gauss":
        x = rng.standard_normal((M, K))
    elif kind == "half_gauss":
        x = 0.5 * rng.standard_normal((M, K))
    elif kind == "correlated":
        base = rng.standard_normal(K)
        noise = rng.standard_normal((M, K))
        x = base[None, :] + 0.1 * noise
    else:
        raise ValueError(f"unknown activation kind {kind!r}")
    return x.astype(np.float32)


def _draw_w(rng: np.random.Generator, kind: str, N: int, K: int) -> np.ndarray:
    w = 0.02 * rng.standard_normal((N, K))
    if kind == "outlier":
        mask = rng.random((N, K)) < 0.01
        w[mask] *= 10.0
    elif kind != "gauss":
        raise ValueError(f"unknown weight kind {kind!r}")
    return w.astype(np.float32)


def make(name: str) -> tuple[np.ndarray, np.ndarray]:
    """Return (X[M][K], W[N][K]) float32 for a named workload."""
    wl = WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    x = _draw_x(rng, wl.x_kind, wl.M, wl.K)
    w = _draw_w(rng, wl.w_kind, wl.N, wl.K)
    return x, w


def make_w(name: str) -> np.ndarray:
    """W only, drawn after X exactly as make() draws it."""
    return make(name)[1]


def random_case(M: int, N: int, K: int, seed: int, x_kind: str = "gauss",
                w_kind: str = "gauss") -> tuple[np.ndarray, np.ndarray]:
    """(X, W) of an arbitrary shape, same recipe as the named workloads."""
    rng = np.random.default_rng(seed)
    return _draw_x(rng, x_kind, M, K), _draw_w(rng, w_kind, N, K)


def coherent_case(M: int, N: int, K: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Sign-coherent (X, W): the magnitudes of a random_case draw, so every
    activation is >= 0 and every weight quantizes to a code >= 8 (every
    product x * w >= 0 and rounding errors of a sum cannot cancel)."""
    x, w = random_case(M, N, K, seed)
    return np.abs(x), np.abs(w)


def integer_case(M: int, N: int, K: int, seed: int, lo: int = -8, hi: int = 8):
    """Integer-valued X in [lo, hi] and raw nibbles in [0, 15], as float32 / uint8.

    Used for the exact special case: with one power-of-two scale for every
    group, every partial sum of the product is an integer multiple of that
    scale far below 2**24, so any summation order is exact in fp32.
    """
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)
    nib = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    return x, nib


def random_words(shape, seed: int) -> np.ndarray:
    """Uniform random int32 words (all bit patterns, negatives included)."""
    rng = np.random.default_rng(seed)
    return rng.integers(-(2 ** 31), 2 ** 31, size=shape, dtype=np.int64).astype(np.int32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
