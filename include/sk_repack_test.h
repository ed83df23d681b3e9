/*
 * sk_repack_test.h -- test hooks of the sk_repack library.
 *
 * Nothing here is used by any entry point of sk_repack.h.  These functions
 * exist so that the layout logic can be checked on a machine without a GPU.
 */
#ifndef SK_REPACK_TEST_H
#define SK_REPACK_TEST_H

#include "sk_repack.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Applies the repack (inverse = 0) or its inverse (inverse = 1) to a HOST copy
 * of a weight's bytes, by running the very index functions the device kernels
 * use (tile interleave by rotations, then the per-tile reorder), one element
 * at a time.  `w` supplies the shape and format (its `data` pointer and
 * `layout` are ignored; `codebook` must follow the format's rule, any non-NULL
 * value will do for SK_W4_CODEBOOK); `host_bytes` must hold `w->bytes` bytes
 * and be 16-byte aligned.  The same validation as sk_repack_w4a8 applies.
 * Every index is bounds-checked; SK_ERR_SHAPE if one ever fell outside the
 * tile or the buffer.
 */
sk_status sk_test_repack_on_host(const sk_weight* w, void* host_bytes, int inverse);

#ifdef __cplusplus
}
#endif

#endif /* SK_REPACK_TEST_H */
