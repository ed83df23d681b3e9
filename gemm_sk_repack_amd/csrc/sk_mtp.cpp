// sk_mtp.cpp -- the adaptive tree-MTP layout planner (host code).
//
// ("Doubling the LLM token rate in ComfyUI", section on adaptive tree MTP.)
// The verification pass has 8 rows: the committed token and 7 drafts, laid out
// as a chain of per-level widths (the first choice of each level continues,
// the runner-ups are leaves).  Per level the planner keeps decayed counts of the
// rank of the accepted token, smooths the measured draft and verify times, and
// every `interval` steps scores the 64 layouts by expected tokens per step over
// verify_ms + depth * draft_ms, moving only for a gain of at least `gain`.
#include <cmath>
#include <cstring>

#include "../../include/sk_mtp.h"

#define SK_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kRows = 7;     // draft rows
constexpr int kRanks = 8;    // 0 = none of the top 7, 1..7

int widths_of(int index, int32_t* w) {
    int d = 0, run = 0;
    for (int row = 1; row <= kRows; ++row) {
        ++run;
        if (row == kRows || ((index >> (row - 1)) & 1)) {
            w[d++] = run;
            run = 0;
        }
    }
    return d;
}

// 1 + sum over levels of P(reach level) * P(rank in 1..w); a level is reached
// through first-choice hits only.  p: [level][8].
double expected_tokens(const double (*p)[kRanks], const int32_t* w, int d) {
    double total = 1.0, reach = 1.0;
    for (int i = 0; i < d; ++i) {
        double hit = 0.0;
        for (int r = 1; r <= w[i]; ++r) hit += p[i][r];
        total += reach * hit;
        reach *= p[i][1];
    }
    return total;
}

}  // namespace

struct sk_mtp_planner {
    double decay, gain;
    int interval;
    double counts[kRows][kRanks];
    double verify_ms, draft_ms;
    bool timed;
    int64_t steps;
    int index;
};

namespace {

// Rank probabilities per level; false when no level has observations yet.
bool probabilities(const sk_mtp_planner* pl, double (*p)[kRanks]) {
    int last = -1;
    for (int i = 0; i < kRows; ++i) {
        double tot = 0.0;
        for (int r = 0; r < kRanks; ++r) tot += pl->counts[i][r];
        if (tot > 0.0) {
            for (int r = 0; r < kRanks; ++r) p[i][r] = pl->counts[i][r] / tot;
            last = i;
        } else if (last >= 0) {
            std::memcpy(p[i], p[last], sizeof(p[i]));
        } else {
            for (int r = 0; r < kRanks; ++r) p[i][r] = 0.0;
        }
    }
    double tot0 = 0.0;
    for (int r = 0; r < kRanks; ++r) tot0 += pl->counts[0][r];
    return tot0 > 0.0;
}

void replan(sk_mtp_planner* pl) {
    double p[kRows][kRanks];
    if (!probabilities(pl, p)) return;
    double scores[64];
    int best = 0;
    for (int b = 0; b < 64; ++b) {
        int32_t w[kRows];
        const int d = widths_of(b, w);
        scores[b] = expected_tokens(p, w, d) / (pl->verify_ms + d * pl->draft_ms);
        if (scores[b] > scores[best]) best = b;
    }
    if (scores[best] >= pl->gain * scores[pl->index]) pl->index = best;
}

}  // namespace

SK_EXPORT sk_status sk_mtp_create(double decay, int32_t interval, double gain, sk_mtp_planner** out) {
    if (!out) return SK_ERR_NULL;
    if (!(decay > 0.0 && decay < 1.0) || interval < 1 || !(gain >= 1.0) || !std::isfinite(gain))
        return SK_ERR_SHAPE;
    sk_mtp_planner* pl = new sk_mtp_planner;
    pl->decay = decay;
    pl->gain = gain;
    pl->interval = interval;
    std::memset(pl->counts, 0, sizeof(pl->counts));
    pl->verify_ms = pl->draft_ms = 0.0;
    pl->timed = false;
    pl->steps = 0;
    pl->index = 63;
    *out = pl;
    return SK_OK;
}

SK_EXPORT void sk_mtp_destroy(sk_mtp_planner* planner) { delete planner; }

SK_EXPORT sk_status sk_mtp_observe(sk_mtp_planner* pl, const int32_t* ranks, int32_t n_levels,
                                   double verify_ms, double draft_ms, int32_t* widths, int32_t* depth) {
    if (!pl || (n_levels > 0 && !ranks)) return SK_ERR_NULL;
    if (n_levels < 0 || n_levels > kRows || !std::isfinite(verify_ms) || !(verify_ms > 0.0) ||
        !std::isfinite(draft_ms) || !(draft_ms > 0.0))
        return SK_ERR_SHAPE;
    for (int i = 0; i < n_levels; ++i)
        if (ranks[i] < 0 || ranks[i] >= kRanks) return SK_ERR_SHAPE;
    for (int i = 0; i < n_levels; ++i) {
        for (int r = 0; r < kRanks; ++r) pl->counts[i][r] *= pl->decay;
        pl->counts[i][ranks[i]] += 1.0;
    }
    const double lam = pl->decay;
    if (!pl->timed) {
        pl->verify_ms = verify_ms;
        pl->draft_ms = draft_ms;
        pl->timed = true;
    } else {
        pl->verify_ms = lam * pl->verify_ms + (1 - lam) * verify_ms;
        pl->draft_ms = lam * pl->draft_ms + (1 - lam) * draft_ms;
    }
    ++pl->steps;
    if (pl->steps % pl->interval == 0) replan(pl);
    int32_t w[kRows];
    const int d = widths_of(pl->index, w);
    if (widths) std::memcpy(widths, w, sizeof(int32_t) * d);
    if (depth) *depth = d;
    return SK_OK;
}

SK_EXPORT sk_status sk_mtp_layout(const sk_mtp_planner* pl, int32_t* index, int32_t* widths, int32_t* depth) {
    if (!pl) return SK_ERR_NULL;
    int32_t w[kRows];
    const int d = widths_of(pl->index, w);
    if (index) *index = pl->index;
    if (widths) std::memcpy(widths, w, sizeof(int32_t) * d);
    if (depth) *depth = d;
    return SK_OK;
}

SK_EXPORT sk_status sk_mtp_layout_of(int32_t index, int32_t* widths, int32_t* depth) {
    if (!widths || !depth) return SK_ERR_NULL;
    if (index < 0 || index >= 64) return SK_ERR_SHAPE;
    *depth = widths_of(index, widths);
    return SK_OK;
}

SK_EXPORT sk_status sk_mtp_accept(const int32_t* widths, int32_t depth, const int32_t* ranks,
                                  int32_t* accepted, int32_t* observed) {
    if (!widths || !ranks || !accepted || !observed) return SK_ERR_NULL;
    if (depth < 1 || depth > kRows) return SK_ERR_SHAPE;
    int sum = 0;
    for (int i = 0; i < depth; ++i) {
        if (widths[i] < 1 || ranks[i] < 0 || ranks[i] >= kRanks) return SK_ERR_SHAPE;
        sum += widths[i];
    }
    if (sum > kRows) return SK_ERR_SHAPE;
    int acc = 0, obs = 0;
    for (int i = 0; i < depth; ++i) {
        ++obs;                                   // this level was drafted and verified
        const int r = ranks[i];
        if (r >= 1 && r <= widths[i]) {
            ++acc;
            if (r != 1) break;                   // a sibling leaf ends the path
        } else {
            break;                               // no candidate matched
        }
    }
    *accepted = acc;
    *observed = obs;
    return SK_OK;
}

SK_EXPORT sk_status sk_mtp_expected_tokens(const double* p, const int32_t* widths, int32_t depth, double* out) {
    if (!p || !widths || !out) return SK_ERR_NULL;
    if (depth < 1 || depth > kRows) return SK_ERR_SHAPE;
    for (int i = 0; i < depth; ++i)
        if (widths[i] < 1 || widths[i] > kRows) return SK_ERR_SHAPE;
    double pp[kRows][kRanks];
    for (int i = 0; i < depth; ++i)
        for (int r = 0; r < kRanks; ++r) pp[i][r] = p[i * kRanks + r];
    *out = expected_tokens(pp, widths, depth);
    return SK_OK;
}

SK_EXPORT sk_status sk_mtp_state(const sk_mtp_planner* pl, double* counts, double* verify_ms, double* draft_ms,
                                 int64_t* steps) {
    if (!pl) return SK_ERR_NULL;
    if (counts) std::memcpy(counts, pl->counts, sizeof(pl->counts));
    if (verify_ms) *verify_ms = pl->verify_ms;
    if (draft_ms) *draft_ms = pl->draft_ms;
    if (steps) *steps = pl->steps;
    return SK_OK;
}
