"""The rounding argument of the kernels' activation quantiser, checked on the CPU.

The kernels form q = rint(fp32(h / sx)) without a division per element: they
round the two exact products h * inv_lo and h * inv_hi, where inv = fp32(1/sx),
inv_lo = fp32(inv * (1 - 2^-22)) and inv_hi = fp32(inv * (1 + 2^-22)), and take
the common value when both round to the same integer (an IEEE division
otherwise).  The argument is that the two products bracket fp32(h / sx).  Here
the rule is evaluated exactly (a product of two float32 values is exact in
float64) on inputs built to sit at or next to half-integer quotients, and on
ordinary random rows, and compared with the oracle's q.
"""

import numpy as np

import oracle as O

F32 = np.float32


def rule(h, sx):
    """(q where the two roundings agree, mask of elements sent to the division)."""
    inv = (F32(1.0) / sx).astype(F32)
    inv_lo = (inv * F32(1.0 - 2.0 ** -22)).astype(F32)
    inv_hi = (inv * F32(1.0 + 2.0 ** -22)).astype(F32)
    h64 = h.astype(np.float64)
    lo = np.rint(h64 * inv_lo.astype(np.float64)[:, None])
    hi = np.rint(h64 * inv_hi.astype(np.float64)[:, None])
    return lo, lo != hi


def check(h):
    q, sx = O.quantize_rows(h)
    lo, split = rule(h, sx)
    agree = ~split
    assert np.array_equal(lo[agree].astype(np.int64), q[agree].astype(np.int64))
    return split.mean()


def test_constants_are_exact():
    assert float(F32(1.0 - 2.0 ** -22)) == 1.0 - 2.0 ** -22
    assert float(F32(1.0 + 2.0 ** -22)) == 1.0 + 2.0 ** -22


def test_near_half_integer_quotients():
    rng = np.random.default_rng(7)
    rows, k = 4096, 256
    amx = rng.uniform(1e-3, 1e3, size=rows).astype(F32)
    sx = (amx / F32(127.0)).astype(F32)
    # quotients at n + 1/2 and a few float32 steps either side of it
    n = rng.integers(-127, 127, size=(rows, k)).astype(np.float64)
    half = (n + 0.5) * sx.astype(np.float64)[:, None]
    steps = rng.integers(-6, 7, size=(rows, k))
    h = half.astype(F32)
    for _ in range(6):
        h = np.where(steps > 0, np.nextafter(h, F32(np.inf)), h)
        h = np.where(steps < 0, np.nextafter(h, F32(-np.inf)), h)
        steps = steps - np.sign(steps)
    h[:, 0] = amx                                    # the row maximum fixes sx
    frac = check(h)
    assert frac > 0.0                                # the band is reached
    assert frac < 0.5


def test_exact_ties_and_power_of_two_scales():
    # sx a power of two: h / sx is exact, and n + 1/2 is an exact tie
    k = 254
    rows = []
    for e in (-20, -3, 0, 5):
        s = 2.0 ** e
        n = np.arange(-127, 127, dtype=np.float64)
        rows.append(((n + 0.5) * s).astype(F32))
    h = np.stack(rows)
    h[:, 0] = (127.0 * 2.0 ** np.array([-20, -3, 0, 5])).astype(F32)
    assert h.shape[1] == k
    check(h)


def test_random_rows_rarely_need_the_division():
    rng = np.random.default_rng(11)
    h = rng.standard_normal((256, 4096)).astype(F32)
    h[::3] *= F32(1e-6)
    h[1::3] *= F32(1e4)
    frac = check(h)
    assert frac < 1e-4
