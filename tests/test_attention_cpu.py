"""Host-side parts of the decode attention (no GPU): the cache layout's host
packing against the layout as include/sk_attention.h states it, argument
validation, and the split planner.

("Doubling the LLM token rate in ComfyUI", section on attention: the cached
prefix is split over many workgroups so that a tiny query fills the GPU.)
"""
import ctypes

import numpy as np
import pytest

import gemm_sk_repack_amd as sk
import synth as S

FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced


def spec_pack(k, v, hkv, length, cap):
    """The cache layout written out from its description, entry by entry."""
    out = np.zeros((hkv, cap // 32, 2, 8, 64, 8), dtype=np.uint16)   # [hk][b][K|V][tile][lane][e]
    for hk in range(hkv):
        for j in range(length):
            b, w = divmod(j, 32)
            kh, r = divmod(w, 16)
            for d in range(128):
                c, rem = divmod(d, 32)
                g, e = divmod(rem, 8)
                out[hk, b, 0, 4 * kh + c, r + 16 * g, e] = k[hk, j, d]
            # V: lane group gv and element ev with key(gv, ev) == w
            if w < 16:
                gv, ev = w // 4, w % 4
            else:
                gv, ev = (w - 16) // 4, 4 + (w - 16) % 4
            for d in range(128):
                out[hk, b, 1, d // 16, d % 16 + 16 * gv, ev] = v[hk, j, d]
    return out.view(np.uint8).reshape(-1)


@pytest.mark.parametrize("hkv,length,cap", [(1, 32, 32), (2, 45, 64), (3, 7, 96), (1, 0, 32)])
def test_host_pack_matches_layout_description(hkv, length, cap):
    q, k, v = S.attention_inputs(5 + length, 1, hkv, hkv, max(length, 1))
    k, v = k[:, :length], v[:, :length]
    got = sk.sk_kv_pack_host(k, v, hkv, length, cap)
    want = spec_pack(k, v, hkv, length, cap)
    assert got.size == sk.kv_cache_bytes(hkv, cap)
    np.testing.assert_array_equal(got, want)


def test_key_order_in_v_tile_is_the_score_layout():
    """key(g, e): lane group g holds entries 4g..4g+3 and 16+4g..16+4g+3, i.e.
    the rows a 16x16 matrix accumulator gives lane group g in each half."""
    seen = []
    for g in range(4):
        for e in range(8):
            seen.append(4 * g + e if e < 4 else 16 + 4 * g + e - 4)
    assert sorted(seen) == list(range(32))


def attn(q=FAKE, m=1, hq=32, hkv=8, kv=FAKE, cap=1024, length=100, scale=0.0883883, out=FAKE):
    return sk.LIB.sk_decode_attention(q, m, hq, hkv, kv, cap, length, ctypes.c_float(scale), out, None, 0,
                                      None)


def test_decode_attention_validation():
    assert attn(q=None) == sk.SK_ERR_NULL
    assert attn(kv=None) == sk.SK_ERR_NULL
    assert attn(out=None) == sk.SK_ERR_NULL
    assert attn(m=0) == sk.SK_ERR_SHAPE
    assert attn(m=9) == sk.SK_ERR_SHAPE
    assert attn(hq=30, hkv=8) == sk.SK_ERR_SHAPE
    assert attn(hkv=0) == sk.SK_ERR_SHAPE
    assert attn(cap=1000) == sk.SK_ERR_SHAPE
    assert attn(length=1025) == sk.SK_ERR_SHAPE
    assert attn(m=4, length=3) == sk.SK_ERR_SHAPE
    assert attn(scale=0.0) == sk.SK_ERR_SHAPE
    assert attn(scale=float("inf")) == sk.SK_ERR_SHAPE
    assert attn(scale=float("nan")) == sk.SK_ERR_SHAPE
    assert attn(m=8, hq=72, hkv=8) == sk.SK_ERR_UNSUPPORTED     # 8 rows x 9 heads per group > 64
    assert attn(hq=1024, hkv=1024) == sk.SK_ERR_UNSUPPORTED      # more KV heads than supported
    assert attn(cap=1 << 23) == sk.SK_ERR_UNSUPPORTED            # a longer cache than supported
    assert attn(q=FAKE + 8) == sk.SK_ERR_ALIGN
    assert attn(kv=FAKE + 4) == sk.SK_ERR_ALIGN
    assert attn(out=FAKE + 4) == sk.SK_ERR_ALIGN


def test_kv_append_validation():
    ap = sk.LIB.sk_kv_append
    assert ap(None, 8, 64, 0, 1, FAKE, FAKE, None) == sk.SK_ERR_NULL
    assert ap(FAKE, 8, 64, 0, 1, None, FAKE, None) == sk.SK_ERR_NULL
    assert ap(FAKE, 0, 64, 0, 1, FAKE, FAKE, None) == sk.SK_ERR_SHAPE
    assert ap(FAKE, 8, 60, 0, 1, FAKE, FAKE, None) == sk.SK_ERR_SHAPE
    assert ap(FAKE, 8, 64, 60, 5, FAKE, FAKE, None) == sk.SK_ERR_SHAPE
    assert ap(FAKE, 8, 64, -1, 1, FAKE, FAKE, None) == sk.SK_ERR_SHAPE
    assert ap(FAKE, 8, 64, 0, 0, FAKE, FAKE, None) == sk.SK_ERR_SHAPE
    assert ap(FAKE + 2, 8, 64, 0, 1, FAKE, FAKE, None) == sk.SK_ERR_ALIGN
    assert ap(FAKE, 8, 64, 0, 1, FAKE + 2, FAKE, None) == sk.SK_ERR_ALIGN


def test_pack_host_validation():
    buf = np.zeros(16, dtype=np.uint16)
    out = np.zeros(16384, dtype=np.uint8)
    p = sk.LIB.sk_kv_pack_host
    assert p(None, buf.ctypes.data, 1, 0, 32, out.ctypes.data) == sk.SK_ERR_NULL
    assert p(buf.ctypes.data, buf.ctypes.data, 1, 33, 32, out.ctypes.data) == sk.SK_ERR_SHAPE
    assert p(buf.ctypes.data, buf.ctypes.data, 1, 0, 48, out.ctypes.data) == sk.SK_ERR_SHAPE
    assert p(buf.ctypes.data, buf.ctypes.data, 0, 0, 32, out.ctypes.data) == sk.SK_ERR_SHAPE


@pytest.mark.parametrize("m,hq,hkv,length", [(1, 32, 8, 16384), (8, 32, 8, 16384), (1, 32, 8, 1),
                                              (8, 40, 8, 32768), (3, 8, 1, 100), (1, 4, 4, 4096),
                                              (8, 64, 8, 1 << 20), (2, 2, 1, 33)])
@pytest.mark.parametrize("cus", [256, 80, 1])
def test_plan_covers_the_prefix(m, hq, hkv, length, cus):
    splits, bps = sk.attention_plan(m, hq, hkv, length, cus)
    nblk = -(-length // 32)
    assert 1 <= splits <= 64
    assert 1 <= bps <= nblk
    assert splits * bps >= nblk and (splits - 1) * bps < nblk     # every range non-empty
    assert bps >= min(4, nblk) or splits == 64                     # a block per wave at least


def test_split_override():
    try:
        sk.set_attention_split(3)
        assert sk.attention_plan(1, 32, 8, 32 * 10, 256) == (4, 3)
        sk.set_attention_split(1000)
        assert sk.attention_plan(1, 32, 8, 32 * 10, 256) == (1, 10)
    finally:
        sk.set_attention_split(0)
    with pytest.raises(sk.SkError):
        sk.set_attention_split(-1)


# Plans measured on the MI355X (Hq 32, Hkv 8, 256 units): about one workgroup per
# two units, ranges of at least 8 blocks, and at least 16 for two query tiles
# from 128 blocks on.
@pytest.mark.parametrize("m,length,plan", [
    (1, 2048, (8, 8)), (8, 2048, (8, 8)), (1, 4096, (16, 8)), (8, 4096, (8, 16)),
    (1, 16384, (16, 32)), (8, 16384, (16, 32)), (1, 32768, (16, 64)), (8, 32768, (16, 64)),
])
def test_plan_for_measured_lengths(m, length, plan):
    assert sk.attention_plan(m, 32, 8, length, 256) == plan
