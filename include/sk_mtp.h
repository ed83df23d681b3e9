/*
 * sk_mtp.h -- C ABI of the adaptive tree-MTP layout planner (host code, in the
 * same library, libsk_repack.so); status codes are those of sk_repack.h.
 *
 * Source, cited by page title and section:
 *  [MTP]  "在 ComfyUI 中将 LLM token 速率翻倍" (Doubling the LLM token rate in
 *         ComfyUI), section "自适应树 MTP" (adaptive tree MTP): a verification
 *         pass carries 8 rows, the committed token and 7 drafts; at each draft
 *         level the MTP head's first choice continues the chain and runner-up
 *         choices are kept as sibling leaves (verified, never drafted from); per
 *         draft level an exponentially decayed count of the rank of the accepted
 *         token (first, second, ... or none) and the measured draft and verify
 *         times drive a re-plan every 32 steps that scores all 64 layouts of the
 *         7 draft rows by expected accepted tokens / (verify_ms + depth *
 *         draft_ms) and switches only when the winner is at least 3% better.
 *
 * Readings where [MTP] is silent:
 *  - A layout is a composition of 7 into depth d >= 1 positive widths; level i
 *    drafts the head's top-w_i candidates.  Layout index b in [0, 64) puts a
 *    level boundary after draft row k (k = 1..6) iff bit k-1 of b is set:
 *    b = 0 is one level of width 7, b = 63 the chain of seven.
 *  - A rank is 1..7 (position of the main model's token among the head's
 *    candidates at that level) or 0 (not among the top 7).  At a level, rank
 *    r <= w accepts a draft; only r = 1 continues to the next level.  Tokens
 *    per step = 1 + accepted drafts.
 *  - Counts: each level whose rank a step reveals is updated as
 *    c <- decay * c + onehot(rank); timings t <- decay * t + (1 - decay) * x
 *    (the first sample taken as is).  p_i(r) = c_i[r] / sum(c_i); a level
 *    without observations borrows the deepest shallower level that has some;
 *    with none at all the planner keeps its layout.
 *  - The re-plan runs after every `interval`-th observed step; ties go to the
 *    lower layout index; the initial layout is the chain (index 63).
 *
 * All pointers are HOST pointers.  Every function returns SK_OK or SK_ERR_NULL
 * / SK_ERR_SHAPE on bad arguments (nothing is changed then).  A planner is
 * owned by the caller (sk_mtp_create / sk_mtp_destroy) and is not thread-safe.
 * All arithmetic is IEEE double in a fixed order.
 */
#ifndef SK_MTP_H
#define SK_MTP_H

#include <stdint.h>

#include "sk_repack.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sk_mtp_planner sk_mtp_planner;

/* New planner [MTP]: decay in (0, 1) (0.95 usual), interval >= 1 steps (32),
 * gain >= 1 (1.03).  *out receives the planner. */
sk_status sk_mtp_create(double decay, int32_t interval, double gain, sk_mtp_planner** out);

/* Frees a planner (NULL is ignored). */
void sk_mtp_destroy(sk_mtp_planner* planner);

/*
 * One verified step [MTP]: ranks[0 .. n_levels) are the ranks the verify pass
 * revealed for draft levels 1 .. n_levels (0..7 each, 0 <= n_levels <= 7),
 * verify_ms and draft_ms the step's measured phase times (finite, > 0; the
 * draft time is per level).  Updates the counts and timings, counts the step
 * and re-plans on every interval-th step.  The layout to use next is written to
 * widths[0 .. *depth) (widths: 7 entries; either output may be NULL).
 */
sk_status sk_mtp_observe(sk_mtp_planner* planner, const int32_t* ranks, int32_t n_levels,
                         double verify_ms, double draft_ms, int32_t* widths, int32_t* depth);

/* The current layout: its index and widths[0 .. *depth) (any output may be NULL). */
sk_status sk_mtp_layout(const sk_mtp_planner* planner, int32_t* index, int32_t* widths, int32_t* depth);

/* Widths of layout `index` (0..63) into widths[0 .. *depth). */
sk_status sk_mtp_layout_of(int32_t index, int32_t* widths, int32_t* depth);

/* Tree verification of one step [MTP]: for ranks[0 .. depth) (0..7) under the
 * layout widths[0 .. depth), the accepted drafts and the number of levels whose
 * rank the pass reveals (the visited levels, the first miss included). */
sk_status sk_mtp_accept(const int32_t* widths, int32_t depth, const int32_t* ranks,
                        int32_t* accepted, int32_t* observed);

/* Expected tokens per step (1 + expected accepted drafts) of a layout given
 * per-level rank probabilities p[level * 8 + rank] (rank 0 = none). */
sk_status sk_mtp_expected_tokens(const double* p, const int32_t* widths, int32_t depth, double* out);

/* The planner's state: counts[level * 8 + rank] (56 doubles), smoothed timings
 * (0 before the first step) and observed steps (any output may be NULL). */
sk_status sk_mtp_state(const sk_mtp_planner* planner, double* counts, double* verify_ms,
                       double* draft_ms, int64_t* steps);

#ifdef __cplusplus
}
#endif

#endif /* SK_MTP_H */
