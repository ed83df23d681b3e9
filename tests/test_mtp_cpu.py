"""The library's tree-MTP planner (host code behind include/sk_mtp.h) against
the oracle: the same layouts, acceptance, expectations, counts, timings and the
same sequence of layout decisions on long synthetic runs.

("Doubling the LLM token rate in ComfyUI", section on adaptive tree MTP.)
Every quantity is IEEE double computed in the same order on both sides, so the
comparisons are exact.
"""
import ctypes

import numpy as np
import pytest

import gemm_sk_repack_amd as sk
from oracle import mtp as T


def test_layouts_match():
    for b in range(64):
        assert sk.mtp_layout_of(b) == T.layout_of(b)


def test_accept_matches_on_every_small_case():
    rng = np.random.default_rng(1)
    for b in range(64):
        w = T.layout_of(b)
        for _ in range(40):
            ranks = [int(x) for x in rng.integers(0, 8, size=len(w))]
            if rng.random() < 0.5:
                ranks = [1] * len(w)
                ranks[int(rng.integers(len(w)))] = int(rng.integers(0, 8))
            assert sk.mtp_accept(w, ranks) == T.accept(w, ranks)


def test_expected_tokens_match():
    rng = np.random.default_rng(2)
    for b in range(64):
        w = T.layout_of(b)
        p = [list(rng.dirichlet(np.ones(8))) for _ in range(len(w))]
        assert sk.mtp_expected_tokens(p, w) == T.expected_tokens_by_levels(p, w)


def regime_ranks(rng, kind, depth_limit=7):
    """Synthetic per-level ranks of the main model's token: 'code' (first choice
    usually right), 'creative' (first choice often wrong, the right token mostly
    in the top 3), 'mixed' (switches every 200 steps)."""
    if kind == "code":
        probs = [0.04, 0.86, 0.06, 0.02, 0.01, 0.005, 0.003, 0.002]
    else:
        probs = [0.15, 0.35, 0.25, 0.13, 0.05, 0.03, 0.02, 0.02]
    return [int(rng.choice(8, p=probs)) for _ in range(depth_limit)]


@pytest.mark.parametrize("kind", ["code", "creative", "mixed"])
@pytest.mark.parametrize("decay,interval,gain", [(0.95, 32, 1.03), (0.8, 8, 1.0), (0.99, 32, 1.1)])
def test_planner_runs_identically(kind, decay, interval, gain):
    rng = np.random.default_rng(hash((kind, interval)) % 2 ** 32)
    lib = sk.MtpPlanner(decay, interval, gain)
    ref = T.Planner(decay, interval, gain)
    switches = 0
    prev = ref.index
    for step in range(1200):
        k = kind if kind != "mixed" else ("code" if (step // 200) % 2 == 0 else "creative")
        ranks_all = regime_ranks(rng, k)
        widths = T.layout_of(ref.index)
        _, observed = T.accept(widths, ranks_all)
        ranks = ranks_all[:observed]
        verify = 10.0 + float(rng.normal(0, 0.3))
        draft = 1.0 + float(rng.normal(0, 0.05))
        w_lib = lib.observe(ranks, verify, draft)
        w_ref = ref.observe(ranks, verify, draft)
        assert w_lib == w_ref, step
        assert lib.index == ref.index
        switches += ref.index != prev
        prev = ref.index
    counts, v, d, steps = lib.state()
    assert counts == ref.counts and v == ref.verify_ms and d == ref.draft_ms and steps == 1200
    if kind == "mixed" and (decay, interval, gain) == (0.95, 32, 1.03):
        assert switches >= 2          # with the page's settings it follows the regime changes


def test_planner_prefers_depth_for_code_and_breadth_for_creative():
    """The page: predictable output favours depth (long chains accepted whole),
    creative writing favours breadth (the right token is usually in the top 3)."""
    for kind, check in (("code", lambda w: len(w) >= 5), ("creative", lambda w: w[0] >= 2)):
        rng = np.random.default_rng(7)
        pl = sk.MtpPlanner()
        w = [1] * 7
        for _ in range(320):
            ranks_all = regime_ranks(rng, kind)
            _, observed = T.accept(w, ranks_all)
            w = pl.observe(ranks_all[:observed], 10.0, 1.0)
        assert check(w), (kind, w)


def test_validation():
    h = ctypes.c_void_p()
    assert sk.LIB.sk_mtp_create(ctypes.c_double(1.0), 32, ctypes.c_double(1.03), ctypes.byref(h)) == sk.SK_ERR_SHAPE
    assert sk.LIB.sk_mtp_create(ctypes.c_double(0.9), 0, ctypes.c_double(1.03), ctypes.byref(h)) == sk.SK_ERR_SHAPE
    assert sk.LIB.sk_mtp_create(ctypes.c_double(0.9), 32, ctypes.c_double(0.5), ctypes.byref(h)) == sk.SK_ERR_SHAPE
    assert sk.LIB.sk_mtp_create(ctypes.c_double(0.9), 32, ctypes.c_double(1.03), None) == sk.SK_ERR_NULL
    pl = sk.MtpPlanner()
    bad = (ctypes.c_int32 * 2)(1, 9)
    assert sk.LIB.sk_mtp_observe(pl._h, bad, 2, ctypes.c_double(1.0), ctypes.c_double(1.0), None, None) == sk.SK_ERR_SHAPE
    ok = (ctypes.c_int32 * 1)(1)
    assert sk.LIB.sk_mtp_observe(pl._h, ok, 8, ctypes.c_double(1.0), ctypes.c_double(1.0), None, None) == sk.SK_ERR_SHAPE
    assert sk.LIB.sk_mtp_observe(pl._h, ok, 1, ctypes.c_double(0.0), ctypes.c_double(1.0), None, None) == sk.SK_ERR_SHAPE
    assert sk.LIB.sk_mtp_observe(pl._h, None, 1, ctypes.c_double(1.0), ctypes.c_double(1.0), None, None) == sk.SK_ERR_NULL
    assert pl.state()[3] == 0                      # nothing changed by the rejected calls
    w = (ctypes.c_int32 * 7)()
    d = ctypes.c_int32()
    assert sk.LIB.sk_mtp_layout_of(64, w, ctypes.byref(d)) == sk.SK_ERR_SHAPE
    assert sk.LIB.sk_mtp_accept((ctypes.c_int32 * 2)(4, 4), 2, (ctypes.c_int32 * 2)(1, 1),
                                ctypes.byref(d), ctypes.byref(d)) == sk.SK_ERR_SHAPE      # 8 rows
