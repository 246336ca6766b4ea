"""CPU checks of how far apart the activations of one row may lie on each
limb-based path, and where the tolerance ends.

Every matrix-core path carries an fp32 activation x as two fp16 limbs of
x' = x * 2^e, with the largest magnitude of some block of the row scaled into
[2^14, 2^15).  The blocks differ:

* the split-precision family (``w4a16_gemm_split``, ``_split_packed``, the
  grouped GEMM, ``w4a16_gemm_repacked`` and ``w4a16_gemm_small_packed``) takes
  one exponent per row (per row and K slice on the small-M kernel) and keeps
  the low limb unscaled: hi = f16(x'), lo = f16(x' - hi);
* the decode GEMV (one exponent per row and group of 32), the skinny kernel
  and the large-M matrix-core tile (per row and pair of groups) carry the low
  limb times 2^11:
  lo = f16((x' - hi) * 2^11), away from the fp16 subnormals.

These tests emulate each representation in NumPy from that statement (no code
of the HIP path), form Y = sum_k rep(x_k) * w_k in fp64 so that only the
representation error remains, and check it against the oracle's tolerance
|dY| <= 1e-5 * sum |x w| + 1e-6.  The worst case puts a large activation on a
zero weight: it sets the exponent but adds nothing to sum |x w|.
"""

import numpy as np

import oracle


def block_exponent(mx):
    """e with mx * 2^e in [2^14, 2^15); 0 for a zero maximum."""
    mx = np.asarray(mx, np.float64)
    e = np.zeros(mx.shape, np.int64)
    ok = mx > 0
    _, E = np.frexp(mx[ok])
    e[ok] = 15 - E
    return e


def rep_row_unscaled(x):
    """Per-row exponent, low limb unscaled (the split-precision family)."""
    x = np.asarray(x, np.float32).astype(np.float64)
    e = block_exponent(np.max(np.abs(x), axis=-1))[..., None]
    xs = np.ldexp(x, e)
    hi = xs.astype(np.float16).astype(np.float64)
    lo = (xs - hi).astype(np.float16).astype(np.float64)
    return np.ldexp(hi + lo, -e)


def rep_block_scaled(x, block):
    """Exponent per row and block of `block` k, low limb carried x2^11 (the
    decode GEMV with block 32, the skinny kernel and the large-M matrix-core
    tile with block 64)."""
    x = np.asarray(x, np.float32).astype(np.float64)
    M, K = x.shape
    xb = x.reshape(M, K // block, block)
    e = block_exponent(np.max(np.abs(xb), axis=-1))[..., None]
    xs = np.ldexp(xb, e)
    hi = xs.astype(np.float16).astype(np.float64)
    lo = ((xs - hi) * 2048.0).astype(np.float16).astype(np.float64)
    return np.ldexp(hi + lo * 2.0 ** -11, -e).reshape(M, K)


def far_apart_case(ratio_log2, seed=0, M=4, N=48, K=256):
    """Rows of N(0,1) activations, each with one entry 2^ratio_log2 times the
    row's scale on a k whose weights are all zero."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    big_k = rng.integers(0, K, M)
    W = rng.standard_normal((N, K)) * 0.02
    for m in range(M):
        X[m, big_k[m]] = 2.0 ** ratio_log2
    W[:, np.unique(big_k)] = 0.0
    X = X.astype(np.float32)
    qw, sc = oracle.quantize(W.astype(np.float32))
    return X, qw, sc


def worst_ratio(rep, X, qw, sc):
    Wd = oracle.dequantize(qw, sc).astype(np.float64)
    Y = rep @ Wd.T
    return oracle.compare(Y, X, qw, sc)["max_ratio"]


def test_row_unscaled_limbs_error_bound():
    """Split family: |x - rep(x)| <= max(2^-22 |x|, 2^-39 max|x_row|)."""
    rng = np.random.default_rng(1)
    x = (rng.uniform(1, 2, (500, 256)) * rng.choice([-1, 1], (500, 256))
         * np.exp2(rng.integers(-50, 1, (500, 256)))).astype(np.float32)
    r = rep_row_unscaled(x)
    xd = x.astype(np.float64)
    mx = np.max(np.abs(xd), axis=1, keepdims=True)
    assert np.all(np.abs(r - xd) <= np.maximum(2.0 ** -22 * np.abs(xd), 2.0 ** -39 * mx))
    # the 22-bit part holds down to about 2^-17 of the row maximum
    near = np.abs(xd) >= mx * 2.0 ** -17
    assert np.all(np.abs(r - xd)[near] <= 2.0 ** -22 * np.abs(xd)[near])


def test_block_scaled_limbs_error_bound():
    """GEMV and skinny kernel: |x - rep(x)| <= max(2^-22 |x|, 2^-50 max|x_block|)."""
    rng = np.random.default_rng(2)
    x = (rng.uniform(1, 2, (500, 256)) * rng.choice([-1, 1], (500, 256))
         * np.exp2(rng.integers(-60, 1, (500, 256)))).astype(np.float32)
    for block in (32, 64):
        r = rep_block_scaled(x, block)
        xd = x.astype(np.float64)
        mx = np.repeat(np.max(np.abs(xd).reshape(500, -1, block), axis=-1), block, axis=1)
        assert np.all(np.abs(r - xd) <= np.maximum(2.0 ** -22 * np.abs(xd), 2.0 ** -50 * mx))


def test_split_family_holds_rows_spanning_2pow20():
    X, qw, sc = far_apart_case(20)
    assert worst_ratio(rep_row_unscaled(X), X, qw, sc) < 0.5


def test_split_family_limit_rows_spanning_2pow30():
    """The documented limit: a row whose entries span 2^30, its largest entry
    on a zero weight, leaves the tolerance on the per-row-exponent paths."""
    X, qw, sc = far_apart_case(30)
    assert worst_ratio(rep_row_unscaled(X), X, qw, sc) > 1.0


def test_block_exponent_paths_hold_rows_spanning_2pow30():
    """The same rows stay inside the tolerance with an exponent per group (the
    decode GEMV) or per pair of groups (the skinny kernel, the large-M tile)."""
    X, qw, sc = far_apart_case(30)
    for block in (32, 64):
        assert worst_ratio(rep_block_scaled(X, block), X, qw, sc) < 0.5
