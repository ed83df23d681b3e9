"""The GEMM launch planner on the host: every plan the library would launch is
inside the kernel's assumptions, and the work it assigns covers every
(tile, super-block) of the weight exactly once."""

import itertools

import numpy as np
import pytest

import gemm_sk_repack_amd as sk

NW = 16

SHAPES = [
    # n, k, g, fmt
    (1024, 1024, 32, 0), (6144, 4096, 32, 0), (4096, 4096, 32, 0), (24576, 4096, 32, 0),
    (4096, 12288, 32, 0), (12288, 4096, 64, 2), (151936, 4096, 32, 0), (7168, 5120, 32, 0),
    (5120, 5120, 32, 0), (34816, 5120, 32, 0), (5120, 17408, 32, 0), (17, 256, 64, 0),
    (5, 128, 128, 0), (1000, 512, 32, 0), (300, 1024, 64, 2), (12288, 4096, 16, 1),
    (2048, 12288, 32, 1),
]


@pytest.mark.parametrize("n,k,g,fmt", SHAPES)
@pytest.mark.parametrize("m", range(1, 9))
@pytest.mark.parametrize("pro", [sk.PRO_NONE, sk.PRO_RMSNORM, sk.PRO_SWIGLU])
def test_plan_within_kernel_assumptions(n, k, g, fmt, m, pro):
    p = sk.gemm_plan(n, k, g, fmt, m, prologue=pro)
    assert p["status"] == sk.SK_OK, p
    T, KB = (n + 15) // 16, k // 128
    S = p["S"]
    assert 1 <= S <= 32 and KB % S == 0
    assert p["KBs"] == KB // S and p["KS"] == k // S
    assert p["P"] == S * p["R"] and p["P"] <= 256 and 1 <= p["R"] <= T
    ept = p["ept"]
    if fmt == sk.SK_W4_CODEBOOK:
        # the codebook runs the MFMA path at every M; 32 without a prologue
        assert ept == (32 if pro == sk.PRO_NONE else 16) and not p["wide"]
    elif m == 1 and pro == sk.PRO_NONE:
        # v_dot4: 16, or 24 in the wide instances where that saves K-slices
        assert ept == (24 if p["wide"] else 16)
        if p["wide"] and S == 1:
            assert k > 16 * 64 * NW
    elif m == 1 or pro == sk.PRO_SWIGLU or (pro == sk.PRO_RMSNORM and fmt != 0):
        assert ept == 16 and not p["wide"]
    elif pro == sk.PRO_RMSNORM:
        # 40 activations with RMSNorm only in the one-slice instances, and only
        # where 16 would need a K-split
        assert ept == (40 if p["wide"] else 16)
        if p["wide"]:
            assert S == 1 and k > 16 * 64 * (NW // m)
    else:
        assert ept == (40 if p["wide"] else 32)
        if p["wide"] and S == 1:
            # the 40-activation instances run only where they save K-slices
            assert k > 32 * 64 * (NW // m)
    # waves per activation row: as many as the slice needs, at most NW / M
    assert p["WPR"] == min(NW // m, -(-p["KS"] // (ept * 64)))
    assert p["KS"] // ept <= p["WPR"] * 64                 # the slice fits the registers
    assert p["TW"] * p["KW"] <= NW and p["TW"] * m * 16 <= NW * 64
    # k-parts: spw super-blocks each, one more for the first srem (K-split only)
    assert p["spw"] * p["KW"] + p["srem"] == p["KBs"] and 0 <= p["srem"] < p["KW"]
    assert S > 1 or p["srem"] == 0
    assert p["lds"] <= 150 * 1024
    # LDS: q (int8, or bf16 after the codebook's 64-byte level table), the wave
    # partials' two halves, and for RMSNorm the slice's gamma
    KS = p["KS"]
    kwp = 4 if p["KW"] <= 4 else 8 if p["KW"] <= 8 else 16   # k-parts padded for the epilogue reads
    red = 2 * p["TW"] * m * 16 * kwp * 4
    gam = 4 * KS if pro == sk.PRO_RMSNORM else 0
    if fmt == sk.SK_W4_CODEBOOK:
        assert p["lds"] == 64 + m * (2 * KS + 64) + red + gam
    else:
        fix = 256 * 12 * 4                                   # the quantiser's list of chunks to redo
        assert p["lds"] == m * (KS + 32) + red + gam + fix
    # register-pipeline depth: 4 for the codebook; 4-bit weights without a
    # prologue take 4 where that pads fewer slots than 5 (at M >= 2: a tenth fewer)
    if fmt == sk.SK_W4_CODEBOOK:
        assert p["pipe"] == 4
    elif fmt == sk.SK_W4_SYM and pro == sk.PRO_NONE:
        assert p["pipe"] in (4, 5)
    else:
        assert p["pipe"] == 5
    if m == 1 and k <= 16384:
        assert S == 1                                        # no cross-slice merge at M = 1
    assert p["part_floats"] == (T * S * m * 16 if S > 1 else 0)


def covered(n, k, m, p):
    """Simulate the kernel's work assignment; count visits per (tile, super-block)."""
    T, KB = (n + 15) // 16, k // 128
    seen = np.zeros((T, KB), dtype=np.int64)
    tq, trem = T // p["R"], T % p["R"]
    for blk in range(p["P"]):
        s, r = blk // p["R"], blk % p["R"]
        t0 = r * tq + min(r, trem)
        t1 = t0 + tq + (1 if r < trem else 0)
        ntile = t1 - t0
        jn = (ntile + p["TW"] - 1) // p["TW"]
        for wv in range(NW):
            tg, kw = wv // p["KW"], wv % p["KW"]
            if tg >= p["TW"] or (p["S"] > 1 and wv == NW - 1):
                continue
            spw_w = p["spw"] + (1 if kw < p["srem"] else 0)
            kwo = kw * p["spw"] + min(kw, p["srem"])
            for i in range(jn * spw_w):
                t = t0 + tg + (i // spw_w) * p["TW"]
                if t >= t1:
                    continue
                kb = s * p["KBs"] + kwo + i % spw_w
                seen[t, kb] += 1
    return seen


@pytest.mark.parametrize("n,k,g,fmt", [s for s in SHAPES if s[0] <= 34816])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_work_covers_every_superblock_once(n, k, g, fmt, m):
    p = sk.gemm_plan(n, k, g, fmt, m)
    assert np.all(covered(n, k, m, p) == 1)


@pytest.mark.parametrize("n,k,m", [(5120, 17408, 8), (5120, 17408, 6), (4096, 12288, 8), (4096, 12288, 4),
                                   (1000, 17408, 8), (12288, 4096, 8)])
def test_uneven_k_parts_cover_every_superblock_once(n, k, m):
    """K-split plans may give the first srem k-parts one super-block more; the
    27B-class down projection at M = 8 (34 super-blocks per slice) then runs 15
    waves (5 tile groups x 3 k-parts) instead of 10."""
    p = sk.gemm_plan(n, k, 32, sk.SK_W4_SYM, m)
    assert np.all(covered(n, k, m, p) == 1)
    if (n, k, m) == (5120, 17408, 8):
        assert (p["S"], p["TW"], p["KW"], p["spw"], p["srem"]) == (4, 5, 3, 11, 1), p


@pytest.mark.parametrize("cus", [1, 7, 64, 80, 256, 304])
def test_plans_for_other_cu_counts(cus):
    for (n, k, g, fmt), m in itertools.product(SHAPES[:6], (1, 8)):
        p = sk.gemm_plan(n, k, g, fmt, m, cus)
        assert p["status"] == sk.SK_OK
        assert p["P"] <= max(cus, p["S"]) and np.all(covered(n, k, m, p) == 1)


def test_forced_split_hook_validates():
    with pytest.raises(sk.SkError):
        sk.set_split(33)
    with pytest.raises(sk.SkError):
        sk.set_split(-1)
    sk.set_split(0)


# Plans measured on the MI355X: the wide instances where they remove or halve the
# K-split (27B-class linears at M >= 6, K = 12288 at M = 3, K = 17408 at M = 1, 2
# and M >= 6), the others where the slice already fits.
@pytest.mark.parametrize("n,k,m,S,wide", [
    (6144, 4096, 8, 1, 0), (4096, 4096, 8, 1, 0), (24576, 4096, 8, 1, 0), (4096, 12288, 8, 4, 0),
    (4096, 12288, 3, 1, 1), (4096, 12288, 2, 1, 0), (7168, 5120, 8, 1, 1), (5120, 5120, 6, 1, 1),
    (34816, 5120, 8, 1, 1), (7168, 5120, 5, 1, 0), (5120, 17408, 8, 4, 1), (5120, 17408, 2, 1, 1),
    (5120, 17408, 1, 1, 1), (4096, 12288, 1, 1, 0),
])
def test_wide_budget_where_measured_faster(n, k, m, S, wide):
    p = sk.gemm_plan(n, k, 32, 0, m)
    assert (p["S"], p["wide"]) == (S, wide), p


@pytest.mark.parametrize("n,k,m,pipe", [
    (7168, 5120, 1, 5), (7168, 5120, 8, 5), (34816, 5120, 1, 4), (34816, 5120, 8, 5),
    (5120, 17408, 1, 5), (5120, 17408, 8, 4), (6144, 4096, 1, 4), (6144, 4096, 8, 4),
    (24576, 4096, 1, 4), (4096, 12288, 1, 4),
])
def test_pipeline_depth_where_measured_faster(n, k, m, pipe):
    """27B-class shapes (5 or 17 super-blocks per wave): 5 slots, except gate+up at
    M = 1 (a 15-wave split of 8) and down at M = 8 (k-parts of 12/11/11); 9B-class
    (4, 6 or 8): 4."""
    p = sk.gemm_plan(n, k, 32, sk.SK_W4_SYM, m)
    assert p["pipe"] == pipe, p


@pytest.mark.parametrize("m,wide", [(1, 0), (4, 0), (5, 1), (8, 1)])
def test_rmsnorm_one_slice_budget(m, wide):
    """RMSNorm + the 9B-class QKV projection: one K-slice at every M."""
    p = sk.gemm_plan(6144, 4096, 32, 0, m, prologue=sk.PRO_RMSNORM)
    assert (p["S"], p["wide"]) == (1, wide), p

