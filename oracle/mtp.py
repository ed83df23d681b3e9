"""CPU oracle for the adaptive tree-MTP layout planner.

TEST INFRASTRUCTURE ONLY.  Only the tests and the CPU-baseline leg of the
benchmark may import this module.  It shares no code with the library and
imports nothing from it.

Source: "在 ComfyUI 中将 LLM token 速率翻倍" (Doubling the LLM token rate in
ComfyUI), section "自适应树 MTP" (adaptive tree MTP).  A verification pass
carries 8 rows: the committed token and 7 draft tokens.  At every draft level
the MTP head's first choice continues the chain; a few runner-up choices at that
level are kept as sibling leaves (verified, never drafted from).  The planner
keeps, per draft level, an exponentially decayed count of the rank at which the
accepted token sat (first, second, ... or none), times the draft and verify
phases, and every 32 steps scores all 64 layouts of the 7 draft rows as a chain
of per-level widths by expected accepted tokens per step (from the conditional
hit probabilities) divided by verify_ms + depth * draft_ms, switching only when
the winner is at least 3% better.

Readings where the page is silent (also listed in the design notes):

* A layout is a composition of 7 into d >= 1 positive widths (w_1, ..., w_d):
  level i drafts the head's top-w_i candidates.  Layout index b in [0, 64) puts
  a level boundary after draft row k (k = 1..6) iff bit k-1 of b is set, so
  b = 0 is one level of width 7 and b = 63 the chain of seven.
* Ranks are 1..7; rank 0 stands for "not among the head's top 7".  At a level,
  a rank r <= w accepts the token; only r = 1 continues to the next level.
* Tokens per step = 1 + accepted drafts (the verify pass always yields the main
  model's own next token after the accepted prefix).
* Decayed counts: at every step, each level whose rank was observed that step
  is updated as c <- lam * c + onehot(rank); other levels are unchanged.
  lam = 0.95 by default.
* Probabilities p_i(r) = c_i[r] / sum(c_i).  A level with no observations yet
  borrows the deepest shallower level that has some; with none at all the
  planner keeps its layout.
* Timings are smoothed the same way: t <- lam * t + (1 - lam) * sample, the
  first sample taken as is.
* Re-planning happens after every 32nd observed step; ties in score go to the
  lower layout index; the switch threshold is score(best) >= 1.03 * score(now).
* The initial layout is the chain of seven (index 63).
"""

from __future__ import annotations

import itertools

DRAFT_ROWS = 7
RANKS = 8            # index 0 = none of the top 7, 1..7 = rank


def layout_of(index: int) -> list[int]:
    """Widths of layout `index` (bit k-1 set: a level boundary after draft row k)."""
    assert 0 <= index < 64
    widths, run = [], 0
    for row in range(1, DRAFT_ROWS + 1):
        run += 1
        if row == DRAFT_ROWS or (index >> (row - 1)) & 1:
            widths.append(run)
            run = 0
    return widths


def all_layouts() -> list[list[int]]:
    return [layout_of(b) for b in range(64)]


def accept(widths, ranks):
    """Tree verification of one step: returns (accepted drafts, levels whose rank
    the verify pass revealed).  ranks[i] is the rank at level i+1 (0 = none)."""
    accepted = 0
    observed = 0
    for i, w in enumerate(widths):
        observed += 1                      # this level was drafted and verified
        r = ranks[i]
        if 1 <= r <= w:
            accepted += 1
            if r != 1:
                break                      # a sibling leaf: nothing hangs below it
        else:
            break                          # no candidate matched: the step ends here
    return accepted, observed


def expected_tokens(p, widths) -> float:
    """Expected tokens per step: 1 + E[accepted drafts], by summing accept() over
    every combination of per-level ranks weighted by the product of the levels'
    rank probabilities p[i][r] (levels treated as independent given the chain)."""
    d = len(widths)
    total = 0.0
    for ranks in itertools.product(range(RANKS), repeat=d):
        pr = 1.0
        for i, r in enumerate(ranks):
            pr *= p[i][r]
            if pr == 0.0:
                break
        if pr == 0.0:
            continue
        acc, _ = accept(widths, ranks)
        total += pr * acc
    return 1.0 + total


def expected_tokens_by_levels(p, widths) -> float:
    """The same expectation walked level by level: a step reaches level i+1
    only through a first-choice hit at level i; at a reached level any rank up
    to the width adds one accepted draft.  Used by the planner (the sum over
    every rank combination above grows as 8^depth)."""
    total, reach = 1.0, 1.0
    for i, w in enumerate(widths):
        total += reach * sum(p[i][r] for r in range(1, w + 1))
        reach *= p[i][1]
    return total


class Planner:
    """The planner's state machine, step by step as the page describes it."""

    def __init__(self, decay: float = 0.95, interval: int = 32, gain: float = 1.03):
        self.decay, self.interval, self.gain = decay, interval, gain
        self.counts = [[0.0] * RANKS for _ in range(DRAFT_ROWS)]
        self.verify_ms = None
        self.draft_ms = None
        self.steps = 0
        self.index = 63

    def probabilities(self):
        p, last = [], None
        for i in range(DRAFT_ROWS):
            tot = sum(self.counts[i])
            if tot > 0.0:
                last = [c / tot for c in self.counts[i]]
            p.append(last)
        return p

    def score(self, p, index):
        w = layout_of(index)
        return expected_tokens_by_levels(p, w) / (self.verify_ms + len(w) * self.draft_ms)

    def observe(self, ranks, verify_ms, draft_ms):
        for i, r in enumerate(ranks):
            for k in range(RANKS):
                self.counts[i][k] *= self.decay
            self.counts[i][r] += 1.0
        lam = self.decay
        self.verify_ms = verify_ms if self.verify_ms is None else lam * self.verify_ms + (1 - lam) * verify_ms
        self.draft_ms = draft_ms if self.draft_ms is None else lam * self.draft_ms + (1 - lam) * draft_ms
        self.steps += 1
        if self.steps % self.interval == 0:
            p = self.probabilities()
            if p[0] is not None:
                scores = [self.score(p, b) for b in range(64)]
                best = max(range(64), key=lambda b: (scores[b], -b))
                if scores[best] >= self.gain * scores[self.index]:
                    self.index = best
        return layout_of(self.index)
