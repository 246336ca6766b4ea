"""CPU checks of the arithmetic the matrix-core decode GEMV is built on.

The kernel scales each group of 32 activations by 2^e (largest magnitude into
[2^14, 2^15)), splits x' = x * 2^e into fp16 limbs hi = f16(x'),
lo = f16((x' - hi) * 2^11), multiplies them by exact fp16 weight codes (q - 8)
and accumulates in fp32.  These tests emulate that arithmetic in NumPy, from
its statement (no code of the HIP path), and check:

* the limb claims: every activation down to 2^-28 of its group maximum is
  carried to 22 significant bits; smaller ones to an absolute 2^-50 of the
  maximum; weight codes and limb-by-code products are exact;
* that the emulated result meets the tolerance of the fp64 oracle on the
  decode workloads' draws and on groups whose magnitudes lie far apart.
"""

import numpy as np
import pytest

import oracle
import workloads


def group_exponent(mx):
    """e with mx * 2^e in [2^14, 2^15); 0 for zero or non-finite; at most 116
    (the kernel forms 2^(e+11) as a normal fp32 number)."""
    mx = np.asarray(mx, np.float64)
    e = np.zeros(mx.shape, np.int64)
    ok = (mx > 0) & np.isfinite(mx)
    _, E = np.frexp(mx[ok])  # mx = f * 2^E, f in [0.5, 1)
    e[ok] = 15 - E
    return np.minimum(e, 116)


def limbs(x):
    """hi, lo (float16) and e for x of shape [..., 32] (one group per row)."""
    x = np.asarray(x, np.float32)
    e = group_exponent(np.max(np.abs(x), axis=-1))
    xs = np.ldexp(x.astype(np.float64), e[..., None])          # exact scaling
    hi = xs.astype(np.float16)                                  # one RNE rounding
    lo = ((xs - hi.astype(np.float64)) * 2048.0).astype(np.float16)
    return hi, lo, e


def test_limbs_carry_22_bits_down_to_2pow_minus28():
    rng = np.random.default_rng(0)
    # 4000 groups: magnitudes spread over 2^-40 .. 2^40 inside each group
    mant = rng.uniform(1.0, 2.0, (4000, 32)) * rng.choice([-1.0, 1.0], (4000, 32))
    spread = rng.integers(-40, 1, (4000, 32))
    base = rng.integers(-60, 61, (4000, 1))
    x = (mant * np.exp2(spread + base)).astype(np.float32)
    hi, lo, e = limbs(x)
    xs = np.ldexp(x.astype(np.float64), e[:, None])
    back = hi.astype(np.float64) + lo.astype(np.float64) * 2.0 ** -11
    err = np.abs(back - xs)
    mx = np.max(np.abs(xs), axis=1, keepdims=True)
    assert np.all((mx >= 2.0 ** 14) & (mx < 2.0 ** 15))
    big = np.abs(xs) >= mx * 2.0 ** -28
    assert np.all(err[big] <= np.abs(xs[big]) * 2.0 ** -22)
    assert np.all(err[~big] <= (mx * 2.0 ** -50 * np.ones_like(xs))[~big])
    assert np.all(np.isfinite(hi)) and np.all(np.isfinite(lo))


def test_codes_and_products_are_exact():
    q = np.arange(16)
    codes = (q - 8).astype(np.float16)
    assert np.array_equal(codes.astype(np.int64), q - 8)
    rng = np.random.default_rng(1)
    limb = rng.uniform(-2.0 ** 15, 2.0 ** 15, 100000).astype(np.float16)
    c = rng.integers(-8, 8, limb.size).astype(np.float16)
    prod32 = limb.astype(np.float32) * c.astype(np.float32)
    assert np.array_equal(prod32.astype(np.float64), limb.astype(np.float64) * c.astype(np.float64))


def emulate_gemv(X, qweight, scales):
    """The kernel's arithmetic for Y = X . dequant(W)^T, in NumPy: per (row,
    group) the exact fp32 limb products summed in fp32 (hi and lo apart),
    combined as s * 2^-e * (D_hi + 2^-11 D_lo) in fp32, groups summed in fp32."""
    M, K = X.shape
    N = qweight.shape[0]
    G = K // 32
    codes = (oracle.unpack(qweight).astype(np.int64) - 8).astype(np.float32).reshape(N, G, 32)
    Y = np.zeros((M, N), np.float32)
    for m in range(M):
        hi, lo, e = limbs(X[m].reshape(G, 32))
        dh = np.zeros((N, G), np.float32)
        dl = np.zeros((N, G), np.float32)
        for k in range(32):  # fp32 accumulation of exact products, one k at a time
            dh = (dh + codes[:, :, k] * hi[None, :, k].astype(np.float32)).astype(np.float32)
            dl = (dl + codes[:, :, k] * lo[None, :, k].astype(np.float32)).astype(np.float32)
        inv = np.ldexp(np.float32(1.0), -e).astype(np.float32)
        sp = (scales * inv[None, :]).astype(np.float32)
        part = (sp * (dh + dl * np.float32(2.0 ** -11)).astype(np.float32)).astype(np.float32)
        acc = np.zeros(N, np.float32)
        for g in range(G):
            acc = (acc + part[:, g]).astype(np.float32)
        Y[m] = acc
    return Y


@pytest.mark.parametrize("name", ["tiny", "decode_down"])
def test_emulated_arithmetic_meets_the_tolerance(name):
    X, W = workloads.make(name)
    if name == "decode_down":
        W = W[:512]  # a slice of the rows keeps the emulation quick
    qw, sc = oracle.quantize(W)
    v = oracle.compare(emulate_gemv(X, qw, sc), X, qw, sc)
    assert v["ok"], v
    assert v["max_ratio"] < 0.05


def test_emulated_arithmetic_far_apart_groups():
    rng = np.random.default_rng(11)
    M, N, K = 2, 64, 2048
    G = K // 32
    X = rng.standard_normal((M, K)) * np.repeat(np.exp2(rng.integers(-100, 101, (M, G)).astype(float)), 32, axis=1)
    X[0, 32 * 7:32 * 8] *= np.exp2(-rng.integers(0, 27, 32).astype(float))
    X = X.astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qw, sc = oracle.quantize(W)
    v = oracle.compare(emulate_gemv(X, qw, sc), X, qw, sc)
    assert v["ok"], v
