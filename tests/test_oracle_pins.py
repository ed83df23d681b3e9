"""Pins of the CPU oracle against facts outside itself (hand-derived examples,
closed forms, invariants, brute force, float64 references within bounds).

Runs on the CPU only.
"""

import itertools

import numpy as np
import pytest

import oracle as O
import synth as S
from conftest import load_golden

F32 = np.float32


# ----------------------------------------------------------------------------
# canonical decoding
# ----------------------------------------------------------------------------

def test_w4_bytes_fixture():
    g = load_golden("w4_w6_bytes.txt")
    vals = np.array(g["w4_values"][0], dtype=np.int64)[None]
    byts = np.array(g["w4_bytes"][0], dtype=np.uint8)[None]
    assert np.array_equal(O.decode_w4(byts, vals.shape[1]), vals)
    assert np.array_equal(S.pack_w4(vals), byts)


def test_u4_bytes_fixture():
    g = load_golden("w4_w6_bytes.txt")
    vals = np.array(g["u4_values"][0], dtype=np.int64)[None]
    byts = np.array(g["u4_bytes"][0], dtype=np.uint8)[None]
    assert np.array_equal(O.decode_u4(byts, vals.shape[1]), vals)
    assert np.array_equal(S.pack_u4(vals), byts)
    # the same bytes read as W4 are the two's-complement values of the indices
    assert np.array_equal(O.decode_w4(byts, vals.shape[1]), np.where(vals >= 8, vals - 16, vals))


def test_w6_bytes_fixture():
    g = load_golden("w4_w6_bytes.txt")
    vals = np.array(g["w6_values"][0], dtype=np.int64)[None]
    byts = np.array(g["w6_bytes"][0], dtype=np.uint8)[None]
    assert np.array_equal(O.decode_w6(byts, vals.shape[1]), vals)
    assert np.array_equal(S.pack_w6(vals), byts)


def test_bf16_widening_fixture():
    g = load_golden("w4_w6_bytes.txt")
    bits = np.array(g["bf16_bits"][0], dtype=np.uint16)
    assert np.array_equal(O.bf16_to_f32(bits), np.array(g["bf16_f32"][0], dtype=F32))
    # rounding to bf16 then widening is within half a bf16 ulp (2^-8 relative)
    x = S.activations(7, 4, 256)
    w = O.bf16_to_f32(S.to_bf16_bits(x))
    assert np.all(np.abs(w - x) <= np.abs(x) * 2.0 ** -8)


def test_w4_exhaustive_positions():
    # every value at both nibble positions decodes back
    vals = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], dtype=np.int64)
    assert np.array_equal(O.decode_w4(S.pack_w4(vals), 2), vals)
    u = np.array([[a, b] for a in range(16) for b in range(16)], dtype=np.int64)
    assert np.array_equal(O.decode_u4(S.pack_u4(u), 2), u)


def test_w6_exhaustive_positions():
    rng = np.random.default_rng(0)
    for r in range(4):
        vals = rng.integers(-32, 32, size=(64, 4))
        vals[:, r] = np.arange(-32, 32)
        assert np.array_equal(O.decode_w6(S.pack_w6(vals), 4), vals)


def test_split_canonical_roundtrip():
    for fmt, k, g in [(0, 256, 32), (2, 256, 64), (1, 128, 16)]:
        vals, s, buf = S.make_weight(fmt, 24, k, g, 11, 12)
        v2, s2 = O.split_canonical(buf, fmt, 24, k, g)
        assert np.array_equal(v2, vals.astype(np.int64))
        assert np.array_equal(s2.view(np.uint32), s.view(np.uint32))
        assert buf.size == S.weight_bytes(fmt, 24, k, g)


def test_shape_rules_fixture():
    g = load_golden("shape_rules.txt")
    for key, fmt in (("w4", 0), ("w6", 2)):
        for k, grp, ok in g[key]:
            assert O.shape_ok(fmt, k, grp) == bool(ok), (key, k, grp)


# ----------------------------------------------------------------------------
# quantiser
# ----------------------------------------------------------------------------

def test_quant_example_a_ties_to_even():
    g = load_golden("quant_examples.txt")
    q, sx = O.quantize_rows(np.array(g["a_x"], dtype=F32))
    assert sx[0] == F32(g["a_sx"][0][0])
    assert q.tolist() == g["a_q"]


def test_quant_example_b():
    g = load_golden("quant_examples.txt")
    q, sx = O.quantize_rows(np.array(g["b_x"], dtype=F32))
    assert int(sx.view(np.uint32)[0]) == g["b_sx_bits"][0][0]
    assert q.tolist() == g["b_q"]


def test_quant_properties():
    h = S.activations(3, 8, 4096) * F32(3.0)
    q, sx = O.quantize_rows(h)
    assert np.all(np.abs(q).max(axis=1) == 127)
    err = np.abs(sx[:, None].astype(np.float64) * q - h)
    assert np.all(err <= sx[:, None] * (0.5 + 2.0 ** -18))
    # sign is kept wherever q is nonzero
    nz = q != 0
    assert np.all(np.sign(q[nz]) == np.sign(h[nz]))


def test_quant_zero_and_constant_rows():
    h = np.zeros((3, 64), F32)
    h[1, :] = -2.5
    h[2, 5] = 1e-30                      # a tiny (normal) absmax still gives 127
    q, sx = O.quantize_rows(h)
    assert sx[0] == 0 and np.all(q[0] == 0)
    assert np.all(q[1] == -127)
    assert q[2, 5] == 127 and np.count_nonzero(q[2]) == 1


def test_quant_example_e_subnormal_scales():
    g = load_golden("quant_examples.txt")
    u = 2.0 ** -149
    for key in ("e1", "e2"):
        x = (np.array(g[key + "_x_units"], dtype=np.float64) * u).astype(F32)
        assert np.array_equal(x[0].astype(np.float64) / u, np.array(g[key + "_x_units"][0]))  # exact
        q, sx = O.quantize_rows(x)
        assert float(sx[0]) == g[key + "_sx_units"][0][0] * u
        assert q.tolist() == g[key + "_q"]


def test_quant_power_of_two_scaling_exact():
    # scaling a row by 2^j scales sx by 2^j and leaves q unchanged (all exact)
    h = S.activations(5, 4, 512)
    q0, s0 = O.quantize_rows(h)
    for j in (-20, -3, 5, 40):
        q1, s1 = O.quantize_rows((h * F32(2.0 ** j)).astype(F32))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, (s0 * F32(2.0 ** j)).astype(F32))


# ----------------------------------------------------------------------------
# exp and prologues
# ----------------------------------------------------------------------------

def test_sk_expf_against_float64():
    x = np.linspace(-87.0, 88.5, 400001).astype(F32)
    e = O.sk_expf(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(F32)).astype(np.float64)
    assert np.max(np.abs(e - ref) / ulp) < 1.5


def test_sk_expf_special_values():
    e = O.sk_expf(np.array([0.0, 89.0, 1000.0, -104.0, -1000.0, -100.0, 1.0], F32))
    assert e[0] == F32(1.0)
    assert np.isinf(e[1]) and np.isinf(e[2])
    assert e[3] == 0 and e[4] == 0
    assert 0 < e[5] < np.finfo(F32).tiny                        # subnormal region
    assert abs(float(e[5]) - np.exp(-100.0)) <= 2.0 ** -149
    assert abs(float(e[6]) - np.e) <= float(np.spacing(F32(np.e)))


def test_rmsnorm_closed_forms():
    k = 1024
    gam = S.gamma(9, k)
    # x == 2, eps = 0: mean square 4, sqrt 2, r = 0.5 exactly -> h == gamma
    h = O.prologue_rmsnorm(np.full((1, k), 2.0, F32), gam, 0.0)
    assert np.array_equal(h[0], gam)
    # x == c, gamma == 1: all h equal, so q is +-127 everywhere
    h = O.prologue_rmsnorm(np.full((2, k), -0.37, F32), np.ones(k, F32), 1e-6)
    assert np.all(h == h[0, 0])
    q, _ = O.quantize_rows(h)
    assert np.all(q == -127)


def test_rmsnorm_against_float64():
    x = S.activations(21, 8, 4096)
    gam = S.gamma(22, 4096)
    h = O.prologue_rmsnorm(x, gam, 1e-6).astype(np.float64)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt(np.mean(x64 ** 2, axis=1, keepdims=True) + 1e-6) * gam
    # 5 fp32 roundings after an exact fp64 sum: a few ulp at most
    assert np.all(np.abs(h - ref) <= 4 * np.abs(ref) * 2.0 ** -24 + 1e-30)


def test_swiglu_closed_forms_and_float64():
    g = S.activations(31, 4, 2048) * F32(4.0)
    u = S.activations(32, 4, 2048)
    assert np.all(O.prologue_swiglu(np.zeros_like(g), u) == 0)
    assert np.all(O.prologue_swiglu(g, np.zeros_like(u)) == 0)
    h = O.prologue_swiglu(g, u).astype(np.float64)
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    ref = g64 / (1.0 + np.exp(-g64)) * u64
    assert np.all(np.abs(h - ref) <= 6 * np.abs(ref) * 2.0 ** -24 + 1e-37)
    # very negative gate: e^-g overflows to inf, silu is -0
    big = O.prologue_swiglu(np.array([[-200.0, -95.0]], F32), np.array([[3.0, -2.0]], F32))
    assert np.all(big == 0)


# ----------------------------------------------------------------------------
# partials and output
# ----------------------------------------------------------------------------

def test_example_c_partials_and_output():
    g = load_golden("quant_examples.txt")
    x = np.array(g["c_x"], dtype=F32)
    q, sx = O.quantize_rows(x)
    assert q.tolist() == g["c_q"]
    assert sx[0] == F32(g["c_sx"][0][0])
    w = np.array([g["c_w0"][0], g["c_w1"][0]], dtype=np.int64)
    s = np.array([g["c_s0"][0], g["c_s1"][0]], dtype=F32)
    p = O.group_partials(w, q, 8)
    assert p.reshape(-1).tolist() == g["c_p"][0]
    y = O.output(p, s, sx)
    assert np.array_equal(y[0], float(sx[0]) * np.array(g["c_y_over_sx"][0]))
    # the same through the canonical buffer
    buf = S.canonical_buffer(S.pack_w4(w), s)
    ref = O.reference(0, buf, 2, 16, 8, x)
    assert np.array_equal(ref["P"], p) and np.array_equal(ref["Y"], y)


def test_partials_brute_force_tiny():
    rng = np.random.default_rng(1)
    for (m, n, k, gsz) in [(1, 3, 16, 4), (3, 5, 32, 8), (2, 4, 64, 16)]:
        w = rng.integers(-8, 8, size=(n, k))
        q = rng.integers(-127, 128, size=(m, k))
        p = O.group_partials(w, q, gsz)
        for mi, ni, j in itertools.product(range(m), range(n), range(k // gsz)):
            acc = 0
            for kk in range(j * gsz, (j + 1) * gsz):
                acc += int(w[ni, kk]) * int(q[mi, kk])
            assert p[mi, ni, j] == acc


def test_all_ones_closed_form():
    n, k, g = 6, 256, 32
    w = np.ones((n, k), np.int64)
    s = np.ones((n, k // g), F32)
    h = S.activations(41, 3, k)
    ref = O.reference(0, S.canonical_buffer(S.pack_w4(w), s), n, k, g, h)
    q = ref["q"].astype(np.int64)
    assert np.array_equal(ref["P"], np.repeat(q.reshape(3, 1, k // g, g).sum(-1), n, axis=1))
    want = ref["sx"].astype(np.float64)[:, None] * q.sum(1, keepdims=True)
    assert np.array_equal(ref["Y"], np.repeat(want, n, axis=1))


def test_identity_closed_form():
    k, g = 64, 16
    w = np.eye(k, dtype=np.int64)
    s = np.ones((k, k // g), F32)
    for fmt, packed in ((0, S.pack_w4(w)), (2, S.pack_w6(w))):
        h = S.activations(42, 2, k)
        ref = O.reference(fmt, S.canonical_buffer(packed, s), k, k, g, h)
        assert np.array_equal(ref["Y"], ref["sx"].astype(np.float64)[:, None] * ref["q"])


def test_rows_are_independent():
    n, k, g = 40, 512, 32
    _, _, buf = S.make_weight(0, n, k, g, 51, 52)
    h = S.activations(53, 8, k)
    full = O.reference(0, buf, n, k, g, h)
    for mi in range(8):
        one = O.reference(0, buf, n, k, g, h[mi:mi + 1])
        assert np.array_equal(one["Y"][0], full["Y"][mi])
        assert np.array_equal(one["P"][0], full["P"][mi])


def test_scale_power_of_two_and_negation():
    n, k, g = 16, 256, 32
    w = S.weights_int(61, n, k, 4).astype(np.int64)
    w = np.clip(w, -7, 7)
    s = S.scales(62, n, k // g)
    h = S.activations(63, 4, k)
    base = O.reference(0, S.canonical_buffer(S.pack_w4(w), s), n, k, g, h)
    sc = O.reference(0, S.canonical_buffer(S.pack_w4(w), s * F32(8.0)), n, k, g, h)
    assert np.array_equal(sc["Y"], 8.0 * base["Y"])
    neg = O.reference(0, S.canonical_buffer(S.pack_w4(-w), s), n, k, g, h)
    assert np.array_equal(neg["Y"], -base["Y"])


def test_codebook_reduces_to_w4():
    n, k, g = 24, 256, 16
    u = S.codes_u4(71, n, k)
    s = S.scales(72, n, k // g)
    h = S.activations(73, 3, k)
    cb = np.arange(-8, 8, dtype=F32)
    cbr = O.reference(1, S.canonical_buffer(S.pack_u4(u), s), n, k, g, h, cb)
    w4 = O.reference(0, S.canonical_buffer(S.pack_w4(u.astype(np.int64) - 8), s), n, k, g, h)
    assert np.array_equal(cbr["F"], w4["P"].astype(np.float64))
    assert np.array_equal(cbr["Y"], w4["Y"])


@pytest.mark.parametrize("fmt,g", [(0, 32), (2, 64), (1, 16)])
def test_dequant_fallback_bound(fmt, g):
    n, k = 48, 1024
    _, _, buf = S.make_weight(fmt, n, k, g, 81, 82)
    cb = S.codebook(86) if fmt == 1 else None
    h = S.activations(83, 5, k)
    ref = O.reference(fmt, buf, n, k, g, h, cb)
    dense = O.dequant_reference(fmt, buf, n, k, g, h, cb)
    bound = O.dequant_bound(fmt, buf, n, k, g, ref["sx"], cb)
    assert np.all(np.abs(ref["Y"] - dense) <= bound * (1 + 1e-12) + 1e-12)
    # and the bound is not vacuous: the typical error is well inside it
    assert np.median(np.abs(ref["Y"] - dense) / bound) < 0.2


def _fp32_round_exact(fr):
    """Round an exact Fraction to the nearest float32 (ties to even), exactly."""
    from fractions import Fraction
    import math
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    t = a / ulp
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * ulp)


def test_quant_matches_exact_rational_near_half_integers():
    """q is rint of the correctly rounded fp32 quotient, checked with exact
    rational arithmetic at points placed within a few ulp of half-integers,
    where dividing and multiplying by a reciprocal disagree."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    sx = F32(2.7) / F32(127.0)
    base = (rng.integers(-126, 126, size=2000) + 0.5) * float(sx)
    h = np.concatenate([[2.7], (base * (1 + rng.integers(-6, 7, size=2000) * 2.0 ** -24))]).astype(F32)
    q, s = O.quantize_rows(h[None])
    assert s[0] == sx
    for hv, qv in zip(h, q[0]):
        t = _fp32_round_exact(Fraction(float(hv)) / Fraction(float(sx)))
        assert qv == int(max(-127, min(127, round(t)))), hv   # Python round: half to even


def test_rmsnorm_sum_of_squares_is_float64():
    """x = [4096, 1 x 4095]: the exact sum of squares is 2^24 + 4095, which an
    fp32 running sum would lose entirely (each +1 is a tie back to 2^24); the
    mean square must come out as 4097, not 4096."""
    k = 4096
    x = np.ones((1, k), F32)
    x[0, 0] = 4096.0
    h = O.prologue_rmsnorm(x, np.ones(k, F32), 1e-6)
    r = float(h[0, 1])
    assert r != 1.0 / 64
    assert abs(r - 1.0 / np.sqrt(4097.0)) <= 2 * float(np.spacing(F32(r)))
    assert float(h[0, 0]) == 4096.0 * r          # multiplying by 2^12 is exact


# ----------------------------------------------------------------------------
# the normaliser of Y's error (reading of the "max relative error" bound)
# ----------------------------------------------------------------------------

def _example_c():
    g = load_golden("quant_examples.txt")
    x = np.array(g["c_x"], dtype=F32)
    q, sx = O.quantize_rows(x)
    w = np.array([g["c_w0"][0], g["c_w1"][0]], dtype=np.int64)
    return g, x, q, sx, w


def test_output_magnitude_example_c():
    g, x, q, sx, w = _example_c()
    s = np.array([g["c_s0"][0], g["c_s1"][0]], dtype=F32)
    p = O.group_partials(w, q, 8)
    mag = O.output_magnitude(p, s, sx)
    assert np.array_equal(mag[0], float(sx[0]) * np.array(g["c_mag_over_sx"][0]))
    # a negative scale: the normaliser keeps |s * P|, while Y changes sign
    s_neg = np.array([g["c_s0"][0], g["c_s1_neg"][0]], dtype=F32)
    mag_neg = O.output_magnitude(p, s_neg, sx)
    assert np.array_equal(mag_neg[0], float(sx[0]) * np.array(g["c_mag_neg_over_sx"][0]))
    y_neg = O.output(p, s_neg, sx)
    assert y_neg[0, 1] == -float(sx[0]) * 2734.0
    # through the whole-call path the same normaliser is returned
    buf = S.canonical_buffer(S.pack_w4(w), s)
    assert np.array_equal(O.reference(0, buf, 2, 16, 8, x)["mag"], mag)


def test_output_magnitude_closed_forms():
    # all-ones weights and scales: mag = sx * sum_j |sum_{k in j} q|, >= |Y| with
    # equality exactly when every group sum has the row's sign
    n, k, g = 5, 256, 32
    h = S.activations(44, 3, k)
    h[1] = np.abs(h[1])                          # row 1: every q >= 0
    ref = O.reference(0, S.canonical_buffer(S.pack_w4(np.ones((n, k), np.int64)),
                                            np.ones((n, k // g), F32)), n, k, g, h)
    q = ref["q"].astype(np.int64).reshape(3, k // g, g).sum(-1)
    want = ref["sx"].astype(np.float64) * np.abs(q).sum(1)
    assert np.array_equal(ref["mag"], np.repeat(want[:, None], n, axis=1))
    assert np.all(ref["mag"] >= np.abs(ref["Y"]))
    assert np.array_equal(ref["mag"][1], np.abs(ref["Y"][1]))
    # scaling every s by 2^j scales the normaliser by 2^j; zero rows give 0
    h0 = np.zeros((1, k), F32)
    _, _, buf = S.make_weight(0, n, k, g, 45, 46)
    assert np.all(O.reference(0, buf, n, k, g, h0)["mag"] == 0)


def test_codebook_magnitude_example_d():
    g, x, q, sx, _ = _example_c()
    u = np.array(g["d_u"], dtype=np.int64)
    cb = np.array(g["d_cb"][0], dtype=F32)
    s = np.array(g["d_s"], dtype=F32)
    f = O.codebook_partials(u, cb, q, 8)
    assert f.reshape(-1).tolist() == g["d_f"][0]
    assert np.array_equal(O.output(f, s, sx)[0], float(sx[0]) * np.array(g["d_y_over_sx"][0]))
    mag = O.codebook_magnitude(u, cb, q, s, sx, 8)
    assert np.array_equal(mag[0], float(sx[0]) * np.array(g["d_mag_over_sx"][0]))
    # the whole-call path on the canonical buffer gives the same values
    buf = S.canonical_buffer(S.pack_u4(u), s)
    ref = O.reference(1, buf, 1, 16, 8, x, cb)
    assert np.array_equal(ref["F"], f) and np.array_equal(ref["mag"], mag)


def test_codebook_magnitude_reduces_to_integer_form():
    # integer levels -8..7: each |level * q| is |w * q|, so the codebook
    # normaliser is sx * sum_j |s| * sum_k |w q| >= the integer one (|sum| <= sum||)
    n, k, g = 16, 256, 16
    u = S.codes_u4(74, n, k)
    s = S.scales(75, n, k // g)
    h = S.activations(76, 2, k)
    cbr = O.reference(1, S.canonical_buffer(S.pack_u4(u), s), n, k, g, h,
                      np.arange(-8, 8, dtype=F32))
    w = u.astype(np.int64) - 8
    q = cbr["q"].astype(np.int64)
    brute = np.zeros((2, n))
    for mi in range(2):
        for ni in range(n):
            brute[mi, ni] = float(cbr["sx"][mi]) * sum(
                float(s[ni, j]) * sum(abs(int(w[ni, kk]) * int(q[mi, kk])) for kk in range(j * g, (j + 1) * g))
                for j in range(k // g))
    assert np.allclose(cbr["mag"], brute, rtol=1e-14, atol=0)
    w4 = O.reference(0, S.canonical_buffer(S.pack_w4(w), s), n, k, g, h)
    assert np.all(cbr["mag"] >= w4["mag"])
