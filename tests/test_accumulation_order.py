"""CPU emulation of the kernels' fp32 summation orders on sign-coherent inputs.

Every kernel accumulates in fp32 (the pages' choice for fidelity: "The
Silence of Success: A Single Line That Speaks Volumes", section "Assumptions
Embedded in the Code"), so its rounding error grows with the length of its
longest chain of additions.  With every product x*w >= 0 the roundings cannot
cancel, which is the hard case for the tolerance
|dY| <= 1e-5 * sum|x*w| + 1e-6.  These tests replay, in NumPy fp32, the
orders the kernels' headers state (written here from those statements, not
from kernel code), with each product rounded to fp32 before it is added
(more roundings than the matrix instructions make):

* tiled kernel: per 32-row output tile, each matrix instruction adds two
  products (k = 32g + 8v + c and 32g + 8v + 4 + c for instruction 4v + c),
  16 instructions per group; the instructions of 8 groups accumulate from zero
  into block sums (one chain, or two chains that take alternate groups, added
  in chain order) that are then added to the running total; with the K range
  split over waves, the waves' totals are added in wave order;
* matrix-core kernels (split path, grouped, small-M, decode GEMV on packed
  weights): each group's 32 products summed from zero, then one fp32 add of
  the group sum per group into the running total;
* large-M matrix-core tile: each group's 32 products summed from zero, the two
  group sums of a pair of groups added, then one fp32 add of the pair sum per
  pair into the running total;
* fp32 GEMV for long K: two chains of 16 products per group (even and odd k),
  their sum, then groups strided over 512 threads chained per thread, then the
  threads' partial sums added in order.

The K limit the header promises (2^17) must keep each order well inside the
tolerance; an unblocked single chain of instructions over all of K (what the
tiled kernel did before its blocks) fails it there, which is why the blocks
exist.
"""

import numpy as np
import pytest

import workloads
from int4_weight_only_03_amd import binding

f32 = np.float32
K_MAX = 1 << 17


def coherent(K, outputs=96, seed=5):
    """fp32 activations >= 0 and dequantized weights >= 0 of one group-32
    quantization (codes 8..15), one (x, w) row pair per emulated output."""
    x, w = workloads.coherent_case(outputs, outputs, K, seed)
    G = K // 32
    wg = w.reshape(outputs, G, 32)
    s = (wg.max(axis=2) / f32(7)).astype(f32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s[..., None] > 0, np.clip(np.rint(wg / s[..., None]), -8, 7), 0)
    wd = (q.astype(f32) * s[..., None]).astype(f32).reshape(outputs, K)
    return x, wd


def ratio(y, x, w):
    p = x.astype(np.float64) * w.astype(np.float64)
    exact, T = p.sum(axis=1), np.abs(p).sum(axis=1)
    return float(np.max(np.abs(y.astype(np.float64) - exact) / (1e-5 * T + 1e-6)))


def tiled_order(x, w, block_groups, waves=1, chains=1):
    P = (x * w).astype(f32)
    O, K = P.shape
    G = K // 32
    total = np.zeros(O, f32)
    for wv in range(waves):
        g0, g1 = G * wv // waves, G * (wv + 1) // waves
        run = np.zeros(O, f32)
        blk = [np.zeros(O, f32) for _ in range(chains)]
        for g in range(g0, g1):
            c = (g - g0) % chains
            for v in range(4):
                for i in range(4):
                    blk[c] = (blk[c] + P[:, 32 * g + 8 * v + i]).astype(f32)
                    blk[c] = (blk[c] + P[:, 32 * g + 8 * v + 4 + i]).astype(f32)
            if block_groups and ((g - g0) % block_groups == block_groups - 1 or g + 1 == g1):
                for c in range(chains):
                    run = (run + blk[c]).astype(f32)
                    blk[c] = np.zeros(O, f32)
        if not block_groups:
            run = blk[0]
        total = (total + run).astype(f32)
    return total


def group_chain_order(x, w):
    P = (x * w).astype(f32)
    O, K = P.shape
    acc = np.zeros(O, f32)
    for g in range(K // 32):
        d = np.zeros(O, f32)
        for i in range(32):
            d = (d + P[:, 32 * g + i]).astype(f32)
        acc = (acc + d).astype(f32)
    return acc


def pair_chain_order(x, w):
    P = (x * w).astype(f32)
    O, K = P.shape
    G = K // 32
    acc = np.zeros(O, f32)
    for g0 in range(0, G, 2):
        pair = np.zeros(O, f32)
        for g in range(g0, min(g0 + 2, G)):
            d = np.zeros(O, f32)
            for i in range(32):
                d = (d + P[:, 32 * g + i]).astype(f32)
            pair = (pair + d).astype(f32)
        acc = (acc + pair).astype(f32)
    return acc


def gemv_long_order(x, w, threads=512):
    P = (x * w).astype(f32)
    O, K = P.shape
    G = K // 32
    part = np.zeros((O, threads), f32)
    for g in range(G):
        e = np.zeros(O, f32)
        o = np.zeros(O, f32)
        for i in range(16):
            e = (e + P[:, 32 * g + 2 * i]).astype(f32)
            o = (o + P[:, 32 * g + 2 * i + 1]).astype(f32)
        t = g % threads
        part[:, t] = (part[:, t] + (e + o).astype(f32)).astype(f32)
    acc = np.zeros(O, f32)
    for t in range(threads):
        acc = (acc + part[:, t]).astype(f32)
    return acc


def test_header_limit_is_the_emulated_one(lib):
    # the library refuses K above 2^17 and accepts it (M = 0: nothing launched)
    assert lib.w4a16_gemm(None, None, None, None, 0, 8, K_MAX, 32, None) == 0
    assert lib.w4a16_gemm(None, None, None, None, 0, 8, K_MAX + 32, 32, None) == 2


@pytest.mark.parametrize("K", [7168, K_MAX])
def test_tiled_blocks_stay_inside(K):
    x, w = coherent(K)
    assert ratio(tiled_order(x, w, 8), x, w) <= 0.2             # 128 x 128 tiles, one wave
    assert ratio(tiled_order(x, w, 8, waves=8, chains=2), x, w) <= 0.2  # skinny, 8 waves


def test_unblocked_chain_fails_at_the_limit():
    # the reason for the blocks: one chain over all of K leaves the tolerance
    x, w = coherent(K_MAX)
    assert ratio(tiled_order(x, w, 0), x, w) > 1.0


@pytest.mark.parametrize("K", [7168, K_MAX])
def test_group_chain_stays_inside(K):
    x, w = coherent(K)
    assert ratio(group_chain_order(x, w), x, w) <= 0.5


@pytest.mark.parametrize("K", [7168, K_MAX])
def test_pair_chain_stays_inside(K):
    x, w = coherent(K)
    assert ratio(pair_chain_order(x, w), x, w) <= 0.5


def test_long_k_gemv_stays_inside():
    x, w = coherent(K_MAX)
    assert ratio(gemv_long_order(x, w), x, w) <= 0.5
