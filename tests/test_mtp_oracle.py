"""Pins of the tree-MTP planner oracle to things other than itself.

("Doubling the LLM token rate in ComfyUI", section on adaptive tree MTP: 8 rows
= the committed token + 7 drafts; first choices continue the chain, runner-ups
are sibling leaves; per-level decayed rank counts; every 32 steps all 64
layouts are scored by expected accepted tokens / (verify_ms + depth *
draft_ms); a switch needs a 3% gain.)
"""
import math

import numpy as np
import pytest

from oracle import mtp as T


def test_there_are_64_layouts_of_seven_rows():
    lays = T.all_layouts()
    assert len(lays) == 64 == 2 ** 6
    assert len({tuple(w) for w in lays}) == 64
    assert all(sum(w) == 7 and min(w) >= 1 for w in lays)
    assert T.layout_of(0) == [7] and T.layout_of(63) == [1] * 7
    # every composition of 7 appears (brute force over sequences of positive parts)
    comps = set()
    def rec(prefix, left):
        if left == 0:
            comps.add(tuple(prefix))
        for k in range(1, left + 1):
            rec(prefix + [k], left - k)
    rec([], 7)
    assert comps == {tuple(w) for w in lays}


def test_page_example_first_choice_wrong_at_depth_one():
    """The page's example: with a chain, a wrong first choice at depth 1 ends the
    step with only the model's own token even when the runner-up was right; a
    layout that keeps the runner-up as a sibling accepts it."""
    ranks = [2, 1, 1, 1, 1, 1, 1]
    assert T.accept([1] * 7, ranks) == (0, 1)
    assert T.accept([2, 1, 1, 1, 1, 1], ranks[:6]) == (1, 1)     # sibling accepted, no children
    assert T.accept([1] * 7, [1] * 7) == (7, 7)
    assert T.accept([3, 4], [1, 4]) == (2, 2)
    assert T.accept([3, 4], [1, 5]) == (1, 2)
    assert T.accept([3, 4], [0, 1]) == (0, 1)


def random_p(rng, depth):
    p = []
    for _ in range(depth):
        v = rng.dirichlet(np.ones(T.RANKS) * 0.7)
        p.append(list(v))
    return p


def test_level_walk_equals_brute_force_over_rank_combinations():
    rng = np.random.default_rng(3)
    for b in range(64):
        w = T.layout_of(b)
        if len(w) > 4:
            continue                  # 8^depth combinations: keep it fast
        p = random_p(rng, len(w))
        assert math.isclose(T.expected_tokens(p, w), T.expected_tokens_by_levels(p, w), rel_tol=1e-12)


@pytest.mark.parametrize("q", [0.0, 0.3, 0.75, 1.0])
def test_chain_closed_form(q):
    """All levels hit their first choice with probability q: a chain of d levels
    yields 1 + q + q^2 + ... + q^d tokens per step."""
    p = [[1 - q, q, 0, 0, 0, 0, 0, 0]] * 7
    assert math.isclose(T.expected_tokens_by_levels(p, [1] * 7), sum(q ** i for i in range(8)), rel_tol=1e-12)
    assert math.isclose(T.expected_tokens(p[:3], [1, 1, 1]), 1 + q + q * q + q ** 3, rel_tol=1e-12)


def test_single_level_closed_form():
    p = [[0.05, 0.3, 0.25, 0.15, 0.1, 0.07, 0.05, 0.03]]
    for w in range(1, 8):
        assert math.isclose(T.expected_tokens(p, [w]), 1 + sum(p[0][1:w + 1]), rel_tol=1e-12)


def test_decayed_counts_closed_form():
    """n identical observations of rank r at one level leave c[r] = (1 - lam^n) / (1 - lam)."""
    pl = T.Planner(decay=0.9, interval=10 ** 9)
    for n in range(1, 30):
        pl.observe([3], 1.0, 0.1)
        assert math.isclose(pl.counts[0][3], (1 - 0.9 ** n) / (1 - 0.9), rel_tol=1e-12)
        assert pl.counts[1] == [0.0] * 8


def test_replans_only_every_interval_and_with_hysteresis():
    """Build statistics where the best layout beats the current one by a known
    factor; the planner moves only at the 32nd step and only past 3%."""
    # creative-writing-like: first choice often wrong, right token in the top 3
    pl = T.Planner()
    for s in range(31):
        assert pl.observe([2, 1, 1], 10.0, 1.0) == [1] * 7
    w = pl.observe([2, 1, 1], 10.0, 1.0)
    assert w != [1] * 7 and w[0] >= 2                       # moved to a wider first level
    # identical statistics afterwards: nothing better by 3%, so it stays put
    idx = pl.index
    for s in range(64):
        pl.observe([2, 1, 1], 10.0, 1.0)
    assert pl.index == idx


def test_switch_threshold_is_three_percent():
    """At a re-plan the planner moves to the best layout iff its score is at
    least 1.03 times the current layout's (checked on random statistics, with
    the step that triggers the re-plan observing no level)."""
    rng = np.random.default_rng(0)
    moved = stayed = 0
    for trial in range(300):
        pl = T.Planner()
        for i in range(7):
            pl.counts[i] = list(rng.dirichlet(np.ones(T.RANKS) * 0.7) * 10)
        pl.verify_ms, pl.draft_ms = 10.0, float(rng.uniform(0.2, 3.0))
        pl.steps = pl.interval - 1
        p = pl.probabilities()
        scores = [pl.score(p, b) for b in range(64)]
        best = max(range(64), key=lambda b: (scores[b], -b))
        # current layout: one close to the best (within 6%) when there is one
        near = [b for b in range(64) if b != best and scores[best] / scores[b] < 1.06]
        pl.index = int(rng.choice(near)) if near else int(rng.integers(64))
        ratio = scores[best] / scores[pl.index]
        if abs(ratio - 1.03) < 1e-9:
            continue
        before = pl.index
        # the timings are re-smoothed with the same values: unchanged
        pl.observe([], 10.0, pl.draft_ms)
        if ratio >= 1.03:
            assert pl.index == best
            moved += 1
        else:
            assert pl.index == before
            stayed += 1
    assert moved > 10 and stayed > 5
