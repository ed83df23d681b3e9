"""CPU oracle for grouped-query decode attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's ``smoke()`` check and
the CPU-baseline leg of the benchmark may import this module.  It shares no
code with the HIP library and imports nothing from it.

Source: "在 ComfyUI 中将 LLM token 速率翻倍" (Doubling the LLM token rate in
ComfyUI), section "关注 attention!": every fourth layer of the hybrid model is
ordinary grouped-query attention with a KV cache, and its decode kernel takes
one token, or a few MTP draft rows that need causal verification, against the
cached prefix without building a mask.

What it computes, written out plainly (fp64 throughout):

    O[m, h, :] = sum_j softmax_j( scale * <q[m, h], k[h // G, j]> ) * v[h // G, j, :]
                 over the keys j = 0 .. L - M + m

Readings where the page is silent (each one is also listed in the design notes):

* Causal verification rows: the M query rows are the last M positions of the
  sequence and their own keys and values are already in the cache (L entries),
  so row m sees keys 0 .. L - M + m (a causal mask aligned to the bottom-right).
* Grouped-query mapping: Hq = G * Hkv and query head h reads KV head h // G
  (consecutive query heads share a KV head).
* Softmax scale 1 / sqrt(D) unless given.
* q, k and v are bfloat16 (the model's activation type); their values are
  widened exactly, and the output is fp64 here (fp32 on the GPU).

Parity pins (tests/test_attention_oracle.py): a hand-derived two-key example
(tests/golden/attention_examples.txt), PyTorch's own scaled-dot-product
attention in float64 with its lower-right causal mask and grouped-query
expansion, the uniform-key closed form, the one-hot limit, and the invariant
that row m of an M-row call equals a one-row call on the first L - M + m + 1
keys.
"""

from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 numbers given as uint16 bits, as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def visible_keys(length: int, m_rows: int, m: int) -> int:
    """Number of cache entries that verification row m sees (reading above)."""
    return length - m_rows + m + 1


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None) -> np.ndarray:
    """Grouped-query decode attention with causal verification rows, in float64.

    q: [M, Hq, D]; k, v: [Hkv, L, D] (real values, e.g. from ``bf16_bits_to_f64``).
    Returns O [M, Hq, D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m_rows, hq, d = q.shape
    hkv, length, dk = k.shape
    assert v.shape == k.shape and dk == d
    assert hq % hkv == 0 and 1 <= m_rows <= length
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((m_rows, hq, d), dtype=np.float64)
    for m in range(m_rows):
        n_vis = visible_keys(length, m_rows, m)
        for h in range(hq):
            kh = h // group
            s = (k[kh, :n_vis] @ q[m, h]) * scale        # scores of the visible keys
            p = np.exp(s - s.max())                      # softmax numerator, shifted for range
            out[m, h] = (p @ v[kh, :n_vis]) / p.sum()
    return out


def decode_attention_bits(q_bits, k_bits, v_bits, scale: float | None = None) -> np.ndarray:
    """``decode_attention`` on bfloat16 inputs given as uint16 bits."""
    return decode_attention(bf16_bits_to_f64(q_bits), bf16_bits_to_f64(k_bits),
                            bf16_bits_to_f64(v_bits), scale)


def decode_attention_rows(q_bits, k_bits, v_bits, rows, scale: float | None = None) -> np.ndarray:
    """Selected outputs only: ``rows`` is a list of (m, h); returns [len(rows), D].

    Same arithmetic as ``decode_attention`` for each requested (m, h), so large
    caches can be checked on a sample without computing every head.
    """
    m_rows, hq, d = q_bits.shape
    hkv, length, _ = k_bits.shape
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((len(rows), d), dtype=np.float64)
    for i, (m, h) in enumerate(rows):
        n_vis = visible_keys(length, m_rows, m)
        kh = h // group
        qv = bf16_bits_to_f64(q_bits[m, h])
        kk = bf16_bits_to_f64(k_bits[kh, :n_vis])
        vv = bf16_bits_to_f64(v_bits[kh, :n_vis])
        s = (kk @ qv) * scale
        p = np.exp(s - s.max())
        out[i] = (p @ vv) / p.sum()
    return out
