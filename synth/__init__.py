"""Seeded synthetic inputs for the skinny quantized linear.

This module draws random tensors and writes them in the canonical storage
format that the library's repack accepts.  It holds none of the method's
arithmetic (no quantisation, no dot products, no prologue math): it is the one
piece that both the CPU oracle's tests and the GPU path's tests may use, so
that the two sides see the same bytes.

Canonical storage (the input of the repack; the pages name N = output width,
K = input width, G = group size and FP32 scales, "Comfy quantization formats",
section "weight formats"; the bit encodings below are this project's reading,
because the format table did not survive on the page):

* W4 symmetric: ``[N, K/2]`` uint8, row-major.  Element ``k = 2j`` sits in the
  low nibble of byte ``j`` and ``k = 2j+1`` in the high nibble, each a 4-bit
  two's-complement integer in ``[-8, 7]``.
* W6 symmetric: ``[N, 3K/4]`` uint8.  Every 4 consecutive elements of a row
  form one 24-bit little-endian word; element ``4i+r`` occupies bits
  ``6r .. 6r+5``, a 6-bit two's-complement integer in ``[-32, 31]``.
* W4 with codebook: like W4, but each nibble is an unsigned index in
  ``[0, 15]`` into a float32[16] table.
* Scales: ``[N, K/G]`` float32, row-major, stored directly after the packed
  weights in the same buffer.

Every generator takes an explicit seed; the seed recipe used throughout is
``1000*config + 10*layer + tensor_id`` with tensor ids w=0, s=1, x=2, gamma=3,
gate=4, up=5, codebook=6.
"""

from __future__ import annotations

import numpy as np

TENSOR_W, TENSOR_S, TENSOR_X, TENSOR_GAMMA, TENSOR_GATE, TENSOR_UP, TENSOR_CB = range(7)


def seed_of(config: int, layer: int, tensor: int) -> int:
    """Seed recipe: 1000*config + 10*layer + tensor id."""
    return 1000 * config + 10 * layer + tensor


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# raw random values
# ----------------------------------------------------------------------------

def weights_int(seed: int, n: int, k: int, bits: int) -> np.ndarray:
    """Uniform signed integers in [-2^(bits-1), 2^(bits-1)-1], shape [N, K], int8."""
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    return _rng(seed).integers(lo, hi + 1, size=(n, k), dtype=np.int64).astype(np.int8)


def codes_u4(seed: int, n: int, k: int) -> np.ndarray:
    """Uniform unsigned 4-bit codebook indices in [0, 15], shape [N, K], uint8."""
    return _rng(seed).integers(0, 16, size=(n, k), dtype=np.int64).astype(np.uint8)


def scales(seed: int, n: int, kg: int, lo: float = 0.002, hi: float = 0.02) -> np.ndarray:
    """Group scales uniform in [lo, hi), shape [N, K/G], float32."""
    return _rng(seed).uniform(lo, hi, size=(n, kg)).astype(np.float32)


def activations(seed: int, m: int, k: int) -> np.ndarray:
    """Activations N(0, 1), shape [M, K], float32."""
    return _rng(seed).standard_normal(size=(m, k)).astype(np.float32)


def gamma(seed: int, k: int) -> np.ndarray:
    """RMSNorm weight uniform in [0.5, 1.5), shape [K], float32."""
    return _rng(seed).uniform(0.5, 1.5, size=(k,)).astype(np.float32)


def codebook(seed: int) -> np.ndarray:
    """16 sorted N(0, 1) levels, float32."""
    return np.sort(_rng(seed).standard_normal(16)).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits.

    Used to make bf16 activations: the value a bf16 input holds is then exactly
    ``bits << 16`` reinterpreted as float32.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


# ----------------------------------------------------------------------------
# canonical packing (storage format writers)
# ----------------------------------------------------------------------------

def pack_w4(w: np.ndarray) -> np.ndarray:
    """[N, K] ints in [-8, 7] -> [N, K/2] uint8, even k in the low nibble."""
    w = np.asarray(w)
    assert w.ndim == 2 and w.shape[1] % 2 == 0
    assert w.min(initial=0) >= -8 and w.max(initial=0) <= 7
    nib = (w.astype(np.int64) & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def pack_u4(u: np.ndarray) -> np.ndarray:
    """[N, K] unsigned indices in [0, 15] -> [N, K/2] uint8, even k in the low nibble."""
    u = np.asarray(u)
    assert u.ndim == 2 and u.shape[1] % 2 == 0
    assert u.min(initial=0) >= 0 and u.max(initial=0) <= 15
    u = u.astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def pack_w6(w: np.ndarray) -> np.ndarray:
    """[N, K] ints in [-32, 31] -> [N, 3K/4] uint8 (4 elements per 24-bit LE word)."""
    w = np.asarray(w)
    assert w.ndim == 2 and w.shape[1] % 4 == 0
    assert w.min(initial=0) >= -32 and w.max(initial=0) <= 31
    n, k = w.shape
    f = (w.astype(np.int64) & 0x3F).reshape(n, k // 4, 4)
    word = f[..., 0] | (f[..., 1] << 6) | (f[..., 2] << 12) | (f[..., 3] << 18)
    out = np.empty((n, k // 4, 3), dtype=np.uint8)
    out[..., 0] = word & 0xFF
    out[..., 1] = (word >> 8) & 0xFF
    out[..., 2] = (word >> 16) & 0xFF
    return out.reshape(n, 3 * k // 4)


def canonical_buffer(packed: np.ndarray, s: np.ndarray) -> np.ndarray:
    """One uint8 buffer holding the packed weights followed by the float32 scales."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    return np.concatenate([np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1),
                           s.view(np.uint8).reshape(-1)])


# ----------------------------------------------------------------------------
# whole weights
# ----------------------------------------------------------------------------

FMT_W4, FMT_W4_CODEBOOK, FMT_W6 = 0, 1, 2
BITS = {FMT_W4: 4, FMT_W4_CODEBOOK: 4, FMT_W6: 6}


def make_weight(fmt: int, n: int, k: int, g: int, seed_w: int, seed_s: int):
    """Draw one weight tensor and return (values, scales, canonical_buffer).

    ``values`` are the signed integers (W4, W6) or the unsigned codebook
    indices; ``canonical_buffer`` is the uint8 array the repack consumes.
    """
    if fmt == FMT_W4:
        vals = weights_int(seed_w, n, k, 4)
        packed = pack_w4(vals)
    elif fmt == FMT_W6:
        vals = weights_int(seed_w, n, k, 6)
        packed = pack_w6(vals)
    elif fmt == FMT_W4_CODEBOOK:
        vals = codes_u4(seed_w, n, k)
        packed = pack_u4(vals)
    else:
        raise ValueError(f"unknown format {fmt}")
    s = scales(seed_s, n, k // g)
    return vals, s, canonical_buffer(packed, s)


def weight_bytes(fmt: int, n: int, k: int, g: int) -> int:
    """Size of the canonical buffer: N*K*bits/8 + N*(K/G)*4."""
    return n * k * BITS[fmt] // 8 + n * (k // g) * 4


# ----------------------------------------------------------------------------
# decode attention inputs
# ----------------------------------------------------------------------------

TENSOR_Q, TENSOR_K, TENSOR_V = 7, 8, 9


def attention_inputs(seed: int, m: int, hq: int, hkv: int, length: int, d: int = 128,
                     q_scale: float = 1.0):
    """Query rows and a KV cache for grouped-query decode attention, as bf16 bits.

    Returns ``(q, k, v)``: q ``[M, Hq, D]``, k and v ``[Hkv, L, D]`` (logical
    order, one contiguous ``[L, D]`` matrix per KV head), each uint16 bfloat16
    bits of N(0, 1) draws (q multiplied by ``q_scale`` first) rounded to
    nearest-even.  Seeds: ``seed + 7`` (q), ``seed + 8`` (k), ``seed + 9`` (v).
    """
    q = _rng(seed + TENSOR_Q).standard_normal(size=(m, hq, d)).astype(np.float32) * np.float32(q_scale)
    k = _rng(seed + TENSOR_K).standard_normal(size=(hkv, length, d)).astype(np.float32)
    v = _rng(seed + TENSOR_V).standard_normal(size=(hkv, length, d)).astype(np.float32)
    return to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)
