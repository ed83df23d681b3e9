"""GPU parity of the grouped-query decode attention (causal verification rows,
prefix split over workgroups, merge in the same launch) against the fp64
oracle, and of the cache append against the host packing.

("Doubling the LLM token rate in ComfyUI", section on attention.)

Tolerance, from the arithmetic: scores are exact bf16 products summed in fp32
over 128 dimensions; the softmax weights are fp32 and enter the value product
as a bf16 pair hi + lo (relative error <= 2^-17); sums over entries, waves and
ranges are fp32.  Each output element therefore stays within a small multiple
of 2^-17 of A[m, h, d] = sum_j p_j |v_jd| / sum_j p_j (the same attention on
|V|), so the test asks |O - O_ref| <= 1e-4 * A + 1e-7.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
import synth as S

pytestmark = pytest.mark.gpu

import gemm_sk_repack_amd as sk  # noqa: E402

TOL = 1e-4


def assert_attn_close(got, qb, kb, vb, rows=None):
    """got: [M, Hq, 128] (rows None) or [len(rows), 128]; compared with the oracle."""
    vabs = vb & np.uint16(0x7FFF)
    if rows is None:
        ref = A.decode_attention_bits(qb, kb, vb)
        mag = A.decode_attention_bits(qb, kb, vabs)
    else:
        ref = A.decode_attention_rows(qb, kb, vb, rows)
        mag = A.decode_attention_rows(qb, kb, vabs, rows)
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    bound = TOL * mag + 1e-7
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), f"worst at {worst}: got {got[worst]} ref {ref[worst]} bound {bound[worst]}"


def make_cache(kb, vb, length, cap):
    hkv = kb.shape[0]
    host = sk.sk_kv_pack_host(kb[:, :length], vb[:, :length], hkv, length, cap)
    return torch.from_numpy(host).cuda()


def run(qb, kv, hkv, cap, length, bps=0):
    q = torch.from_numpy(qb.view(np.int16)).cuda()
    sk.set_attention_split(bps)
    try:
        out = sk.sk_decode_attention(q, hkv, kv, cap, length)
        torch.cuda.synchronize()
    finally:
        sk.set_attention_split(0)
    return out.cpu().numpy()


def roundup(x, a):
    return (x + a - 1) // a * a


def test_append_matches_host_pack():
    hkv, cap = 3, 128
    _, kb, vb = S.attention_inputs(901, 1, hkv, hkv, 54)
    kv = torch.zeros(sk.kv_cache_bytes(hkv, cap), dtype=torch.uint8, device="cuda")
    for pos, t in ((0, 45), (45, 1), (46, 8)):
        kn = torch.from_numpy(np.ascontiguousarray(kb[:, pos:pos + t].transpose(1, 0, 2)).view(np.int16)).cuda()
        vn = torch.from_numpy(np.ascontiguousarray(vb[:, pos:pos + t].transpose(1, 0, 2)).view(np.int16)).cuda()
        sk.sk_kv_append(kv, hkv, cap, pos, kn, vn)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kv.cpu().numpy(), sk.sk_kv_pack_host(kb, vb, hkv, 54, cap))


@pytest.mark.parametrize("m,hq,hkv,length", [
    (1, 4, 1, 37), (1, 32, 8, 300), (3, 8, 2, 333), (8, 32, 8, 1000), (8, 40, 8, 517),
    (8, 64, 8, 200), (5, 12, 4, 64), (2, 2, 2, 2), (1, 1, 1, 1), (8, 32, 8, 8), (4, 16, 2, 4097)])
def test_parity_planner(m, hq, hkv, length):
    cap = roundup(length, 32) + 32
    qb, kb, vb = S.attention_inputs(1000 + 7 * m + length, m, hq, hkv, length)
    kv = make_cache(kb, vb, length, cap)
    print(f"m={m} hq={hq} hkv={hkv} L={length} plan={sk.attention_plan(m, hq, hkv, length)}", flush=True)
    assert_attn_close(run(qb, kv, hkv, cap, length), qb, kb, vb)


@pytest.mark.parametrize("bps", [1, 2, 3, 5, 8, 1000])
@pytest.mark.parametrize("m,hq,hkv,length", [(1, 32, 8, 777), (8, 32, 8, 777), (6, 30, 6, 250),
                                              (4, 16, 2, 2048), (8, 40, 8, 1100), (8, 64, 8, 1500)])
def test_parity_forced_splits(m, hq, hkv, length, bps):
    cap = roundup(length, 32)
    qb, kb, vb = S.attention_inputs(2000 + m + length, m, hq, hkv, length)
    kv = make_cache(kb, vb, length, cap)
    assert_attn_close(run(qb, kv, hkv, cap, length, bps), qb, kb, vb)


@pytest.mark.parametrize("q_scale", [4.0, 12.0, 30.0])
def test_peaked_scores(q_scale):
    """Scores with a spread of tens to hundreds (log2 units): the running
    maximum moves often and the rescaling decides the result; a reference
    that is not the true row maximum would overflow exp2 here."""
    m, hq, hkv, length = 8, 16, 4, 700
    cap = roundup(length, 32)
    qb, kb, vb = S.attention_inputs(3100, m, hq, hkv, length, q_scale=q_scale)
    kv = make_cache(kb, vb, length, cap)
    for bps in (0, 1, 1000):
        assert_attn_close(run(qb, kv, hkv, cap, length, bps), qb, kb, vb)


def test_entries_past_the_prefix_are_ignored():
    """Cache entries at or past L hold NaN and Inf bit patterns: the output is
    bit-identical to the run with zeros there."""
    m, hq, hkv, length = 8, 32, 8, 301
    cap = roundup(length, 32) + 64
    qb, kb, vb = S.attention_inputs(3200, m, hq, hkv, cap)
    clean = make_cache(kb, vb, length, cap)
    kb2, vb2 = kb.copy(), vb.copy()
    kb2[:, length:] = 0x7FC0            # NaN
    vb2[:, length:] = 0x7F80            # +Inf
    vb2[:, length + 1::2] = 0xFFC1      # NaN
    dirty = torch.from_numpy(sk.sk_kv_pack_host(kb2, vb2, hkv, cap, cap)).cuda()
    for bps in (0, 1, 1000):
        a = run(qb, clean, hkv, cap, length, bps)
        b = run(qb, dirty, hkv, cap, length, bps)
        np.testing.assert_array_equal(a, b)
    assert_attn_close(a, qb, kb[:, :length], vb[:, :length])


def test_deterministic():
    m, hq, hkv, length = 8, 32, 8, 5000
    cap = roundup(length, 32)
    qb, kb, vb = S.attention_inputs(3300, m, hq, hkv, length)
    kv = make_cache(kb, vb, length, cap)
    a = run(qb, kv, hkv, cap, length)
    for _ in range(3):
        np.testing.assert_array_equal(a, run(qb, kv, hkv, cap, length))


def test_decode_step_with_append():
    """The serving order: the cache holds L0 entries, the step appends its M
    new entries (committed token + drafts) and attends over L0 + M."""
    m, hq, hkv, l0 = 8, 32, 8, 1234
    length = l0 + m
    cap = 2048
    qb, kb, vb = S.attention_inputs(3400, m, hq, hkv, length)
    kv = make_cache(kb, vb, l0, cap)
    kn = torch.from_numpy(np.ascontiguousarray(kb[:, l0:].transpose(1, 0, 2)).view(np.int16)).cuda()
    vn = torch.from_numpy(np.ascontiguousarray(vb[:, l0:].transpose(1, 0, 2)).view(np.int16)).cuda()
    sk.sk_kv_append(kv, hkv, cap, l0, kn, vn)
    assert_attn_close(run(qb, kv, hkv, cap, length), qb, kb, vb)


@pytest.mark.parametrize("m", [1, 8])
def test_full_size_sampled(m):
    """The 9B-class layer's attention at a 16384-entry prefix (Hq 32, Hkv 8),
    with the planner's split, checked on sampled (row, head) outputs."""
    hq, hkv, length = 32, 8, 16384
    qb, kb, vb = S.attention_inputs(4000 + m, m, hq, hkv, length)
    kv = make_cache(kb, vb, length, length)
    out = run(qb, kv, hkv, length, length)
    rng = np.random.default_rng(m)
    rows = sorted({(int(rng.integers(m)), int(rng.integers(hq))) for _ in range(12)} | {(m - 1, hq - 1), (0, 0)})
    got = np.stack([out[mm, h] for mm, h in rows])
    assert_attn_close(got, qb, kb, vb, rows)


def test_long_prefix_sampled():
    """A 131072-entry prefix with two KV heads: the planner's largest split (64
    ranges per head, 64 blocks each), checked on sampled (row, head) outputs."""
    m, hq, hkv, length = 8, 8, 2, 131072
    qb, kb, vb = S.attention_inputs(4100, m, hq, hkv, length)
    assert sk.attention_plan(m, hq, hkv, length) == (64, 64)
    kv = make_cache(kb, vb, length, length)
    out = run(qb, kv, hkv, length, length)
    rows = [(0, 0), (7, 7), (3, 4), (5, 1), (6, 6), (1, 3)]
    got = np.stack([out[mm, h] for mm, h in rows])
    assert_attn_close(got, qb, kb, vb, rows)
