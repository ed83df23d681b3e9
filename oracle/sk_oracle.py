"""CPU oracle for the skinny quantized linear  Y[M,N] = dequant(W)[N,K] . int8(X)[M,K]^T.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's ``smoke()`` check and
the CPU-baseline leg of the benchmark may import this module.  It shares no
code with the HIP library and imports nothing from it.

Sources (web pages; cited by title and section):

* "在 ComfyUI 中将 LLM token 速率翻倍" (Doubling the LLM token rate in ComfyUI),
  section "优化线性 Kernel" (optimizing linear kernels): W4A8 / W6A8 weights
  with per-group scales; the activation is quantised to int8 inside the linear
  kernel; RMSNorm or SwiGLU may be folded in front of that quantisation.
* "Comfy 量化格式" (Comfy quantization formats), sections "权重格式" (weight
  formats) and "格式选项" (format options): N is the output width, K the input
  width, G the group size, scales are FP32; W4 with an optional float[16]
  codebook; W6 without one; weights are exported symmetric (no zero point);
  shape rules.  Section "激活与平滑" (activations and smoothing): integer
  formats take float activations and quantise them in the kernel.

Readings where the pages are silent:

* Canonical bit encodings (the format table is missing from the page): see
  ``decode_w4``, ``decode_w6``, ``decode_u4``.
* Activation quantisation is per row (token): a = max|h|, sx = a/127 (fp32
  division), q = clamp(round-half-even(fp32(h/sx)), -127, 127); a row whose
  sx is 0 (all zeros, or an absmax so small that absmax/127 rounds to 0 in
  fp32) gets q = 0: with a zero scale every code dequantises to 0.
* RMSNorm h = (x * r) * gamma with r = 1/sqrt(mean(x^2) + eps); the sum of
  squares in float64, everything else fp32 with each operation rounded once.
* SwiGLU h = (g / (1 + e^-g)) * u with e^x evaluated by ``sk_expf`` below, a
  fixed float32 operation sequence (Cody-Waite reduction + Taylor polynomial)
  so both sides round identically.
* Output accumulation over groups in float64 here (float32 on the GPU).

Parity pins: every function here is checked in tests/test_oracle_pins.py
against hand-derived examples, closed forms, invariants, exhaustive brute
force on tiny inputs, or float64 references within a stated bound.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32


# ----------------------------------------------------------------------------
# canonical weight decoding ("Comfy quantization formats", weight formats)
# ----------------------------------------------------------------------------

def decode_w4(packed: np.ndarray, k: int) -> np.ndarray:
    """[N, K/2] uint8 -> [N, K] int64 in [-8, 7].

    Reading: byte j holds element 2j in its low nibble and 2j+1 in its high
    nibble; a nibble is a 4-bit two's-complement integer.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    out = np.empty((n, k), dtype=np.int64)
    lo = (packed & 0x0F).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    out[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out


def decode_u4(packed: np.ndarray, k: int) -> np.ndarray:
    """[N, K/2] uint8 -> [N, K] int64 unsigned codebook indices in [0, 15]."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    out = np.empty((n, k), dtype=np.int64)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def decode_w6(packed: np.ndarray, k: int) -> np.ndarray:
    """[N, 3K/4] uint8 -> [N, K] int64 in [-32, 31].

    Reading: every 3 bytes form a little-endian 24-bit word holding 4
    consecutive elements, element r of the four at bits 6r..6r+5, each a 6-bit
    two's-complement integer.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    b = packed.reshape(n, k // 4, 3).astype(np.int64)
    word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
    out = np.empty((n, k // 4, 4), dtype=np.int64)
    for r in range(4):
        f = (word >> (6 * r)) & 0x3F
        out[..., r] = np.where(f >= 32, f - 64, f)
    return out.reshape(n, k)


BITS = {0: 4, 1: 4, 2: 6}          # format id -> bits per weight (W4, W4+codebook, W6)


def split_canonical(buf: np.ndarray, fmt: int, n: int, k: int, g: int):
    """Split one canonical buffer into (weight values [N,K] int64, scales [N,K/G] f32).

    The buffer is the packed weights followed directly by the FP32 scales.
    For the codebook format the values are the unsigned indices.
    """
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    wbytes = n * k * BITS[fmt] // 8
    kg = k // g
    assert buf.size == wbytes + n * kg * 4
    wpart = buf[:wbytes].reshape(n, k * BITS[fmt] // 8)
    s = buf[wbytes:].copy().view(np.float32).reshape(n, kg)
    if fmt == 0:
        vals = decode_w4(wpart, k)
    elif fmt == 1:
        vals = decode_u4(wpart, k)
    elif fmt == 2:
        vals = decode_w6(wpart, k)
    else:
        raise ValueError(fmt)
    return vals, s


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 (given as uint16 bits) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# shape rules ("Comfy quantization formats", format options)
# ----------------------------------------------------------------------------

def shape_ok(fmt: int, k: int, g: int) -> bool:
    """The format's shape rules as the page states them (before any backend limits).

    Grouped W4: K divisible by 16 and by G; G at least 4 and either dividing 16
    or a multiple of 16.  W6: K divisible by 32 and G a multiple of 16 (and,
    for whole groups, G dividing K).
    """
    if fmt in (0, 1):
        return k % 16 == 0 and g >= 4 and k % g == 0 and (16 % g == 0 or g % 16 == 0)
    if fmt == 2:
        return k % 32 == 0 and g % 16 == 0 and g > 0 and k % g == 0
    return False


# ----------------------------------------------------------------------------
# exp for the SwiGLU prologue: one fixed float32 sequence
# ----------------------------------------------------------------------------

# Cody & Waite (1980) additive argument reduction with ln 2 split in two parts:
# the high part has few significant bits so n*LN2_HI is exact for |n| < 2^14.
_LOG2E = F32(1.4426950408889634)
_LN2_HI = F32(0.693359375)
_LN2_LO = F32(0.6931471805599453 - 0.693359375)
# Taylor coefficients 1/j! of e^r, j = 0..7 (|r| <= ln2/2 makes the truncation
# error r^8/8! < 6e-9, below half an fp32 ulp of the result).
_TAYLOR = [F32(1.0 / f) for f in (1.0, 1.0, 2.0, 6.0, 24.0, 120.0, 720.0, 5040.0)]


def _pow2_f32(e: np.ndarray) -> np.ndarray:
    """2^e as float32 for integer e in [-126, 127], built from the exponent field."""
    return ((e.astype(np.int64) + 127) << 23).astype(np.uint32).view(np.float32)


def sk_expf(x: np.ndarray) -> np.ndarray:
    """e^x in float32 by a fixed operation sequence (each op rounded once, no FMA).

    1. x >= 89 -> +inf; x <= -104 -> +0 (beyond fp32 range either way).
    2. n = rint(fp32(x * log2 e)).
    3. r = (x - n*LN2_HI) - n*LN2_LO.
    4. p = Horner evaluation of sum_{j<=7} r^j / j!, multiply then add.
    5. result = (p * 2^(n//2)) * 2^(n - n//2)   (the first product is exact).
    """
    x = np.asarray(x, dtype=F32)
    big = x >= F32(89.0)
    small = x <= F32(-104.0)
    xs = np.where(big | small, F32(0.0), x).astype(F32)
    n = np.rint(xs * _LOG2E).astype(F32)
    r = (xs - n * _LN2_HI) - n * _LN2_LO
    p = _TAYLOR[7]
    for c in reversed(_TAYLOR[:7]):
        p = p * r + c
    ni = n.astype(np.int64)
    e1 = ni // 2                      # floor division
    e2 = ni - e1
    res = (p * _pow2_f32(e1)) * _pow2_f32(e2)
    res = np.where(big, F32(np.inf), res)
    res = np.where(small, F32(0.0), res)
    return res.astype(F32)


# ----------------------------------------------------------------------------
# prologues ("Doubling the LLM token rate", optimizing linear kernels)
# ----------------------------------------------------------------------------

def prologue_rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """h = fp32(fp32(x * r) * gamma), r = fp32(1 / fp32(sqrt(fp32(fp32(ss/K) + eps)))).

    ss = sum of x^2 in float64 (each square is exact in float64).
    """
    x = np.asarray(x, dtype=F32)
    gamma = np.asarray(gamma, dtype=F32)
    k = x.shape[1]
    ss = np.sum(x.astype(np.float64) ** 2, axis=1)
    ms = (ss / np.float64(k)).astype(F32)
    d = ms + F32(eps)
    r = F32(1.0) / np.sqrt(d)
    return ((x * r[:, None]) * gamma[None, :]).astype(F32)


def prologue_swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """h = fp32(fp32(g / fp32(1 + sk_expf(-g))) * u)."""
    g = np.asarray(gate, dtype=F32)
    u = np.asarray(up, dtype=F32)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        den = F32(1.0) + sk_expf(-g)
        silu = g / den
    return (silu * u).astype(F32)


# ----------------------------------------------------------------------------
# activation quantisation (in-kernel, per row)
# ----------------------------------------------------------------------------

def quantize_rows(h: np.ndarray):
    """Per-row symmetric int8 quantisation.

    a = max_k |h|; sx = fp32(a / 127); q = clamp(rint(fp32(h / sx)), -127, 127)
    with rint rounding half to even.  A row whose sx is 0 gets q = 0: the
    all-zero row, and a nonzero row with a < 127 * 2^-150, whose quotient
    a/127 rounds to 0 in fp32 (the formula would divide by zero; with a zero
    scale every code dequantises to 0, so 0 is the one consistent code).
    Returns (q int8 [M,K], sx float32 [M]).
    """
    h = np.asarray(h, dtype=F32)
    assert np.all(np.isfinite(h)), "the oracle takes finite activations only"
    a = np.max(np.abs(h), axis=1) if h.shape[1] else np.zeros(h.shape[0], F32)
    sx = (a / F32(127.0)).astype(F32)
    q = np.zeros(h.shape, dtype=np.int8)
    nz = sx > 0
    if np.any(nz):
        t = (h[nz] / sx[nz][:, None]).astype(F32)
        q[nz] = np.clip(np.rint(t), -127, 127).astype(np.int8)
    sx = np.where(nz, sx, F32(0.0)).astype(F32)
    return q, sx


# ----------------------------------------------------------------------------
# per-group integer partials and the output
# ----------------------------------------------------------------------------

def group_partials(w: np.ndarray, q: np.ndarray, g: int) -> np.ndarray:
    """P[m, n, j] = sum_{k in group j} w[n, k] * q[m, k], exact in int64."""
    w = np.asarray(w, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    n, k = w.shape
    m = q.shape[0]
    kg = k // g
    wg = w.reshape(n, kg, g)
    qg = q.reshape(m, kg, g)
    return np.einsum("njk,mjk->mnj", wg, qg)


def codebook_partials(u: np.ndarray, cb: np.ndarray, q: np.ndarray, g: int) -> np.ndarray:
    """F[m, n, j] = sum_{k in group j} cb[u[n, k]] * q[m, k], in float64."""
    lv = np.asarray(cb, dtype=F32).astype(np.float64)[np.asarray(u, dtype=np.int64)]
    n, k = lv.shape
    m = q.shape[0]
    kg = k // g
    return np.einsum("njk,mjk->mnj", lv.reshape(n, kg, g),
                     np.asarray(q, dtype=np.float64).reshape(m, kg, g))


def output(partials: np.ndarray, s: np.ndarray, sx: np.ndarray) -> np.ndarray:
    """Y[m, n] = sx[m] * sum_j s[n, j] * P[m, n, j], evaluated in float64."""
    p = np.asarray(partials, dtype=np.float64)
    s64 = np.asarray(s, dtype=F32).astype(np.float64)
    acc = np.sum(p * s64[None, :, :], axis=2)
    return np.asarray(sx, dtype=F32).astype(np.float64)[:, None] * acc


def output_magnitude(partials: np.ndarray, s: np.ndarray, sx: np.ndarray) -> np.ndarray:
    """sx[m] * sum_j |s[n, j] * P[m, n, j]|: the scale Y's rounding error is measured against.

    Reading of the "max relative error" bound on Y: Y is a signed sum of K/G
    terms and may sit near zero, so the error is normalised by the sum of the
    terms' magnitudes, each |s * P| (the absolute value covers the scale too).
    """
    p = np.abs(np.asarray(partials, dtype=np.float64))
    s64 = np.abs(np.asarray(s, dtype=F32).astype(np.float64))
    return np.asarray(sx, dtype=F32).astype(np.float64)[:, None] * np.sum(p * s64[None], axis=2)


def codebook_magnitude(u, cb, q, s, sx, g: int) -> np.ndarray:
    """Like output_magnitude for the codebook: sx * sum_j |s| * sum_{k in j} |cb[u] * q|.

    The codebook's group sums have no exact integer form, so every product
    cb[u] * q counts with its own magnitude."""
    lv = np.abs(np.asarray(cb, dtype=F32).astype(np.float64)[np.asarray(u, dtype=np.int64)])
    aq = np.abs(np.asarray(q, dtype=np.float64))
    n, k = lv.shape
    m = aq.shape[0]
    kg = k // g
    t = np.einsum("njk,mjk->mnj", lv.reshape(n, kg, g), aq.reshape(m, kg, g))
    return output_magnitude(t, s, sx)


# ----------------------------------------------------------------------------
# whole calls
# ----------------------------------------------------------------------------

def reference(fmt: int, buf: np.ndarray, n: int, k: int, g: int, h: np.ndarray,
              cb: np.ndarray | None = None):
    """Full linear on already-prologued float32 activations h [M, K].

    Returns a dict with q, sx, P (integer formats) or F (codebook), Y (float64)
    and the error scale ``mag`` used to normalise |Y_gpu - Y|.
    """
    vals, s = split_canonical(buf, fmt, n, k, g)
    q, sx = quantize_rows(h)
    if fmt == 1:
        assert cb is not None
        f = codebook_partials(vals, cb, q, g)
        y = output(f, s, sx)
        mag = codebook_magnitude(vals, cb, q, s, sx, g)
        return {"q": q, "sx": sx, "F": f, "Y": y, "mag": mag, "w": vals, "s": s}
    p = group_partials(vals, q, g)
    return {"q": q, "sx": sx, "P": p, "Y": output(p, s, sx),
            "mag": output_magnitude(p, s, sx), "w": vals, "s": s}


def dequant_reference(fmt: int, buf: np.ndarray, n: int, k: int, g: int, h: np.ndarray,
                      cb: np.ndarray | None = None) -> np.ndarray:
    """Dequantise-then-dense in float64 on the UNquantised activations.

    This is the fallback the quantization-format page describes for a format
    whose fast path is disabled; the quantised result must stay within
    ``dequant_bound`` of it.
    """
    vals, s = split_canonical(buf, fmt, n, k, g)
    lv = (np.asarray(cb, dtype=F32).astype(np.float64)[vals] if fmt == 1
          else vals.astype(np.float64))
    wd = lv * np.repeat(s.astype(np.float64), g, axis=1)
    return np.asarray(h, dtype=np.float64) @ wd.T


def dequant_bound(fmt: int, buf: np.ndarray, n: int, k: int, g: int, sx: np.ndarray,
                  cb: np.ndarray | None = None) -> np.ndarray:
    """|Y_quantised - Y_dense| <= sx * (0.5 + 2^-18) * sum_k |s[n, g(k)] * w[n, k]|.

    Each |sx*q_k - h_k| is at most sx*(0.5 + 2^-18): rint moves at most 1/2,
    and fp32(h/sx) is within half an ulp (<= 2^-18 for |h/sx| < 128) of h/sx.
    """
    vals, s = split_canonical(buf, fmt, n, k, g)
    lv = (np.asarray(cb, dtype=F32).astype(np.float64)[vals] if fmt == 1
          else vals.astype(np.float64))
    wabs = np.abs(lv) * np.repeat(s.astype(np.float64), g, axis=1)
    return (np.asarray(sx, dtype=np.float64)[:, None] * (0.5 + 2.0 ** -18)) * wabs.sum(axis=1)[None, :]
