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

/*
 * The launch plan the library would use for a GEMM call with this shape, M,
 * prologue (0 none, 1 RMSNorm, 2 SwiGLU) and compute-unit count (host
 * arithmetic only).  fields[0..14] receive
 * S (K-slices), R (workgroups per slice), P (workgroups), TW (tile groups per
 * workgroup), KW (waves along k), super-blocks per wave per tile,
 * super-blocks per slice, K per slice, waves per activation row, dynamic LDS
 * bytes, workspace floats for slice partials, activations per thread in the
 * prologue (16, 24, 32 or 40), 1 if the kernel instance with the larger activation
 * budget runs (else 0), the register-pipeline depth the wave split was chosen
 * for (slots of weights in flight per wave) and the number of k-parts that take
 * one super-block more than the given count (K-split launches only; else 0).
 * SK_ERR_UNSUPPORTED if no
 * plan exists; SK_ERR_SHAPE for shapes outside the backend's range.
 */
sk_status sk_test_gemm_plan(int n, int k, int group, int format, int m, int prologue, int cus,
                            int64_t* fields);

/* Forces the number of K-slices of later GEMM calls (1..32; 0 restores the
 * automatic choice).  Calls whose K/128 the forced value does not divide, or
 * whose slice does not fit the kernel's layout, return SK_ERR_UNSUPPORTED. */
sk_status sk_test_set_split(int s);

/* Number of polls of a cross-slice exchange slot before a workgroup computes
 * that slice's statistics itself (0 restores the default).  A small value
 * forces the local path, which must give identical results. */
sk_status sk_test_set_spin_limit(int polls);

/* Streaming-read probe, the reference ceiling for the GEMM's weight stream:
 * `grid` workgroups of `threads` threads (64..1024, a multiple of 64) read the
 * device buffer `buf` of `bytes` bytes (16-byte aligned, a multiple of 16) once
 * with 16-byte loads, each workgroup a contiguous share, eight loads in flight
 * per thread, and fold it into one word; `out` (device, 4 bytes) is written only
 * if the fold equals a fixed value, so the reads cannot be elided.  Errors: NULL,
 * SHAPE (bytes < 16 or not a multiple of 16, grid < 1, threads outside
 * 64..1024 or not a multiple of 64), ALIGN, HIP. */
sk_status sk_test_stream_read(const void* buf, int64_t bytes, int grid, int threads,
                              uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SK_REPACK_TEST_H */
