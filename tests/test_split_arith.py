"""The split-bfloat16 arithmetic of the fused E-step kernels, checked on the
CPU with bfloat16 round-to-nearest-even emulated bit by bit: the facts the
kernels' error bound and their statistics accuracy rest on.

* two-part split (logits): x_hi = bf16(x), x_lo = bf16(x - x_hi), with
  x - x_hi exact in float32, leaves |x - x_hi - x_lo| <= 2^-17 |x| (the
  kernels' bound takes 2^-16);
* the three logit passes x_hi w_hi + x_hi w_lo + x_lo w_hi miss x w by at
  most 3.1 * 2^-16 |x w| (the split term of the refinement bound);
* three-part split (statistics): x = x_hi + x_mid + x_lo exactly;
* the six statistics products of order up to two miss r x by at most
  2^-23 (1 + 2^-7) |r x|, the float32 rounding level, while r's parts stay
  normal (r >= 2^-100); below that the miss is under 2^-126 |x|, far below
  what the float32 tile sums resolve.
No GPU and no library: the same steps written out in numpy."""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf16(x):
    """Round float32 values to bfloat16 (nearest, ties to even), returned as
    float32: keep the top 16 bits of the IEEE word after adding 0x7FFF plus
    the lowest kept bit."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def sample(n, seed, lo=-30, hi=30):
    """float32 values with random signs, significands and exponents in
    [2^lo, 2^hi) (normal range, no overflow of products or squares)."""
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(lo, hi, n)
    sign = rng.choice([-1.0, 1.0], n)
    return (sign * mant * np.exp2(expo)).astype(np.float32)


def split2(x):
    h = bf16(x)
    d = (x - h).astype(np.float32)  # float32 subtraction, as in the kernel
    return h, bf16(d), d


def split3(x):
    h = bf16(x)
    r1 = (x - h).astype(np.float32)
    m = bf16(r1)
    r2 = (r1 - m).astype(np.float32)
    return h, m, bf16(r2), r1, r2


def test_bf16_rounding_matches_definition():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: to even (1); 1 + 3 * 2^-8 ties up to 1 + 2^-6
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -1.5, 3.0e38], dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -1.5, 2.0**127 * 1.765625], dtype=np.float32)
    got = bf16(x)
    np.testing.assert_array_equal(got[:5], want[:5])
    # every result has at most 8 significant bits and is the nearest such value
    v = sample(100_000, 1)
    b = bf16(v).astype(np.float64)
    assert np.all((b.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    err = np.abs(v.astype(np.float64) - b)
    assert np.all(err <= np.exp2(np.floor(np.log2(np.abs(v.astype(np.float64)))) - 8) * (1 + 1e-12))


def test_two_part_split_error():
    x = sample(200_000, 2)
    h, l, d = split2(x)
    xd = x.astype(np.float64)
    # x - x_hi is exact in float32
    np.testing.assert_array_equal(d.astype(np.float64), xd - h.astype(np.float64))
    err = np.abs(xd - h.astype(np.float64) - l.astype(np.float64))
    assert np.all(err <= 2.0**-17 * np.abs(xd))
    # the bound is nearly reached, so it is the right one
    assert np.max(err / np.abs(xd)) > 0.99 * 2.0**-17


def test_three_logit_passes_error():
    x, w = sample(200_000, 3, -20, 20), sample(200_000, 4, -20, 20)
    xh, xl, _ = split2(x)
    wh, wl, _ = split2(w)
    f = np.float64
    approx = f(xh) * f(wh) + f(xh) * f(wl) + f(xl) * f(wh)  # each product exact in float32 (8 x 8 bits)
    exact = f(x) * f(w)
    assert np.all(np.abs(exact - approx) <= 3.1 * 2.0**-16 * np.abs(exact))
    for a, b in ((xh, wh), (xh, wl), (xl, wh)):
        p = f(a) * f(b)
        np.testing.assert_array_equal(p, f(np.float32(p)))


def test_three_part_split_is_exact():
    x = sample(300_000, 5)
    h, m, l, r1, r2 = split3(x)
    f = np.float64
    np.testing.assert_array_equal(f(r1), f(x) - f(h))
    np.testing.assert_array_equal(f(r2), f(r1) - f(m))
    np.testing.assert_array_equal(f(l), f(r2))  # the last remainder fits in bfloat16
    np.testing.assert_array_equal(f(h) + f(m) + f(l), f(x))


def test_six_statistics_products_error():
    rng = np.random.default_rng(6)
    r = rng.uniform(0.0, 1.0, 200_000).astype(np.float32)  # responsibilities
    r[:1000] = np.exp(-rng.uniform(0, 80, 1000)).astype(np.float32)
    x = sample(200_000, 7, -12, 12)
    rp, xp = split3(r)[:3], split3(x)[:3]
    f = np.float64
    approx = sum(f(rp[i]) * f(xp[j]) for i in range(3) for j in range(3) if i + j <= 2)
    exact = f(r) * f(x)
    big = r >= 2.0**-100
    assert np.all(np.abs(exact - approx)[big] <= 2.0**-23 * (1 + 2.0**-7) * np.abs(exact)[big])
    assert np.all(np.abs(exact - approx)[~big] <= 2.0**-126 * np.abs(f(x))[~big])
    assert np.any(~big) and np.max(np.abs(exact - approx)[big] / np.abs(exact)[big]) > 2.0**-25
    # one-hot r (the k-means mode): r is exact in bf16, so three passes give r x exactly
    one = np.ones_like(x)
    oh = split3(one)
    assert np.all(f(oh[1]) == 0) and np.all(f(oh[2]) == 0)
    np.testing.assert_array_equal(f(oh[0]) * (f(xp[0]) + f(xp[1]) + f(xp[2])), f(x))
