"""Pins of the decode-attention oracle to things other than itself.

("Doubling the LLM token rate in ComfyUI", section on attention: grouped-query
attention with a KV cache; one token or a few draft rows with causal
verification.)  A dropped scale, a wrong head mapping, an off-by-one in the
causal limit or a transposed operand each fails at least one of these.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

from conftest import load_golden
from oracle import attention as A
import synth as S


def _arr(rows):
    return np.array(rows, dtype=np.float64)


def test_golden_two_keys():
    g = load_golden("attention_examples.txt")
    q = _arr(g["two_q"]).reshape(1, 1, 4)
    k = _arr(g["two_k"]).reshape(1, 2, 4)
    v = _arr(g["two_v"]).reshape(1, 2, 4)
    o = A.decode_attention(q, k, v)
    np.testing.assert_allclose(o.reshape(-1), _arr(g["two_o"]).reshape(-1), rtol=0, atol=1e-15)


def test_golden_causal_rows():
    g = load_golden("attention_examples.txt")
    q = _arr(g["causal_q"]).reshape(2, 1, 4)
    k = _arr(g["causal_k"]).reshape(1, 3, 4)
    v = _arr(g["causal_v"]).reshape(1, 3, 4)
    o = A.decode_attention(q, k, v)
    np.testing.assert_allclose(o.reshape(2, 4), _arr(g["causal_o"]), rtol=0, atol=1e-15)


def test_golden_group_mapping():
    g = load_golden("attention_examples.txt")
    q = _arr(g["groups_q"]).reshape(1, 4, 4)
    k = np.stack([_arr(g["groups_k0"]), _arr(g["groups_k1"])])
    v = np.zeros((2, 3, 4))
    v[0, :, 0] = 1.0
    v[1, :, 1] = 1.0
    o = A.decode_attention(q, k, v)
    np.testing.assert_allclose(o.reshape(4, 4), _arr(g["groups_o"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("m,hq,hkv,length,d,qs", [
    (1, 4, 1, 37, 16, 1.0), (3, 8, 2, 50, 32, 1.0), (8, 32, 8, 70, 128, 1.0),
    (8, 40, 8, 33, 128, 3.0), (5, 6, 3, 5, 8, 0.5), (2, 2, 2, 2, 4, 10.0)])
def test_matches_torch_sdpa_lower_right_causal(m, hq, hkv, length, d, qs):
    """PyTorch's scaled-dot-product attention (float64, CPU) with its own
    lower-right causal bias and grouped-query expansion is an independent
    definition of the same operation."""
    qb, kb, vb = S.attention_inputs(11 * m + length, m, hq, hkv, length, d, qs)
    o = A.decode_attention_bits(qb, kb, vb)
    q = torch.from_numpy(A.bf16_bits_to_f64(qb)).permute(1, 0, 2).unsqueeze(0)
    k = torch.from_numpy(A.bf16_bits_to_f64(kb)).unsqueeze(0)
    v = torch.from_numpy(A.bf16_bits_to_f64(vb)).unsqueeze(0)
    ref = F.scaled_dot_product_attention(q, k, v, attn_mask=causal_lower_right(m, length),
                                         enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_uniform_keys_give_the_mean_of_visible_values():
    """Equal scores make the softmax uniform: row m returns the mean of the
    first L - M + m + 1 value rows."""
    m, hq, hkv, length, d = 4, 4, 2, 11, 8
    rng = np.random.default_rng(5)
    q = rng.standard_normal((m, hq, d))
    k = np.broadcast_to(rng.standard_normal(d), (hkv, length, d)).copy()
    v = rng.standard_normal((hkv, length, d))
    o = A.decode_attention(q, k, v)
    for mm in range(m):
        n_vis = length - m + mm + 1
        for h in range(hq):
            np.testing.assert_allclose(o[mm, h], v[h // 2, :n_vis].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_one_hot_limit():
    """A query aligned with one key and a wide score gap picks that key's value
    up to the weight exp(-gap) of every other key."""
    d, length = 16, 9
    k = np.zeros((1, length, d))
    for j in range(length):
        k[0, j, j] = 1.0
    v = np.random.default_rng(2).standard_normal((1, length, d))
    q = np.zeros((1, 1, d))
    q[0, 0, 6] = 200.0                     # score 200/4 = 50 for key 6, 0 for the rest
    o = A.decode_attention(q, k, v)
    bound = (length - 1) * math.exp(-50.0) * np.abs(v).max() * 2
    np.testing.assert_allclose(o[0, 0], v[0, 6], rtol=0, atol=bound)


def test_row_equals_single_row_call_on_its_prefix():
    """Causal verification: row m of an M-row call is a one-row call on the
    first L - M + m + 1 cache entries."""
    m, hq, hkv, length, d = 6, 8, 4, 25, 32
    qb, kb, vb = S.attention_inputs(77, m, hq, hkv, length, d)
    o = A.decode_attention_bits(qb, kb, vb)
    for mm in range(m):
        n_vis = length - m + mm + 1
        single = A.decode_attention_bits(qb[mm:mm + 1], kb[:, :n_vis], vb[:, :n_vis])
        np.testing.assert_array_equal(o[mm], single[0])


def test_key_order_does_not_matter():
    qb, kb, vb = S.attention_inputs(3, 1, 4, 2, 40, 16)
    perm = np.random.default_rng(9).permutation(40)
    o1 = A.decode_attention_bits(qb, kb, vb)
    o2 = A.decode_attention_bits(qb, kb[:, perm], vb[:, perm])
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)


def test_scale_argument():
    """scale * <q, k> is all that matters: doubling q and halving the scale
    changes nothing; the default scale is 1/sqrt(D)."""
    q, k, v = (A.bf16_bits_to_f64(t) for t in S.attention_inputs(4, 2, 4, 4, 19, 32))
    o1 = A.decode_attention(q, k, v)
    o2 = A.decode_attention(2.0 * q, k, v, scale=0.5 / math.sqrt(32))
    o3 = A.decode_attention(q, k, v, scale=1.0 / math.sqrt(32))
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(o1, o3)


def test_sampled_rows_match_full_call():
    qb, kb, vb = S.attention_inputs(8, 8, 16, 4, 45, 128)
    o = A.decode_attention_bits(qb, kb, vb)
    rows = [(0, 0), (7, 15), (3, 5), (5, 12)]
    got = A.decode_attention_rows(qb, kb, vb, rows)
    for i, (mm, h) in enumerate(rows):
        np.testing.assert_allclose(got[i], o[mm, h], rtol=1e-14, atol=1e-15)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    vals = A.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0
    assert vals[2] == 3.140625
    assert vals[3] == 2.0 ** -133
    assert vals[4] == (2 - 2.0 ** -7) * 2.0 ** 127
