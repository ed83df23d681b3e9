"""The rounding argument of the kernels' activation quantiser, checked on the CPU.

The kernels form q = rint(fp32(h / sx)) without a division per element: they
round the two exact products h * inv_lo and h * inv_hi, where inv = fp32(1/sx),
inv_lo = fp32(inv * (1 - 2^-22)) and inv_hi = fp32(inv * (1 + 2^-22)), and take
the common value when both round to the same integer.  Where they differ, the
element's code comes from the corrected quotient (fp32(h * inv) refined twice by
an FMA residual), and a row whose sx is below 2^-100 takes IEEE division
throughout.  The bracket argument is checked here exactly (a product of two
float32 values is exact in float64) on inputs built to sit at or next to
half-integer quotients, and on ordinary random rows, against the oracle's q.
The whole rule, correction included, is restated in C (tests/quant_rule) and
compared with IEEE division, exhaustively over every float h for a set of
scales and on random scales and elements.
"""

import os
import subprocess

import numpy as np
import pytest

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


# ---------------------------------------------------------------------------
# the whole rule, correction included, in C against IEEE division
# ---------------------------------------------------------------------------

HERE = os.path.dirname(os.path.abspath(__file__))
RULE_SRC = os.path.join(HERE, "quant_rule", "rule_check.c")
RULE_EXE = os.path.join(HERE, os.pardir, "_build", "quant_rule", "rule_check")


def _host_has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.fixture(scope="module")
def rule_check():
    """The checker, built with gcc when missing or older than its source (the
    host's FMA instructions where it has them: glibc's fmaf is exact either
    way, only slower)."""
    exe = os.path.normpath(RULE_EXE)
    if not os.path.exists(exe) or os.path.getmtime(exe) < os.path.getmtime(RULE_SRC):
        os.makedirs(os.path.dirname(exe), exist_ok=True)
        flags = ["-O2", "-std=c99", "-Wall"] + (["-mfma"] if _host_has_fma() else [])
        subprocess.run(["gcc", *flags, "-o", exe, RULE_SRC, "-lm"], check=True)
    return exe, _host_has_fma()


def _run(exe, arg):
    out = subprocess.run([exe, arg], capture_output=True, text=True, timeout=300)
    line = out.stdout.strip().splitlines()[-1]
    checked, corrected, bad = (int(v) for v in line.split()[1::2])
    return out.returncode, checked, corrected, bad, out.stdout


def test_corrected_rule_matches_division_for_every_float_of_hard_scales(rule_check):
    exe, fast = rule_check
    if not fast:
        pytest.skip("no hardware FMA on this host: the exhaustive sweep would take minutes")
    rc, checked, corrected, bad, text = _run(exe, "exhaustive")
    assert rc == 0 and bad == 0, text
    assert checked > 700_000_000          # nine scales, sx/4 <= h <= 127.01 sx each
    assert corrected > 1000               # the correction is exercised, not bypassed


def test_corrected_rule_matches_division_on_random_scales(rule_check):
    exe, fast = rule_check
    rc, checked, corrected, bad, text = _run(exe, "20000000" if fast else "2000000")
    assert rc == 0 and bad == 0, text
    assert corrected > checked // 10      # most of the half-integer neighbourhoods need it
