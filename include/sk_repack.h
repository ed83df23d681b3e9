/*
 * sk_repack.h -- C ABI of the MI355X (gfx950) skinny quantized linear library.
 *
 *   Y[M,N] = dequant(W)[N,K] . int8(h)[M,K]^T ,   M = 1..8,
 *
 * where W is a 4-bit or 6-bit weight with FP32 per-group scales, h is the
 * activation (optionally produced by an RMSNorm or SwiGLU prologue) and int8()
 * is per-row symmetric quantisation done inside the GEMM launch.
 *
 * Sources, cited by page title and section:
 *  [LIN]  "在 ComfyUI 中将 LLM token 速率翻倍" (Doubling the LLM token rate in
 *         ComfyUI), section "优化线性 Kernel" (optimizing linear kernels):
 *         W4A8/W6A8 skinny GEMV/GEMM; weights and their per-group scales
 *         interleaved in the order the kernel consumes them, so each workgroup
 *         streams contiguous memory; the re-layout is done once per model load,
 *         in place, with no extra memory; M up to 8 rows; RMSNorm/SwiGLU folded
 *         into the activation quantisation.
 *  [FMT]  "Comfy 量化格式" (Comfy quantization formats), sections "权重格式"
 *         (weight formats: N, K, G, FP32 scales), "格式选项" (format options:
 *         W4 codebook, W6, symmetric export, shape rules) and "激活与平滑"
 *         (activations: integer formats quantise float input in the kernel).
 *
 * Conventions for every entry point
 *  - All pointers except `sk_weight*` itself are DEVICE pointers to memory the
 *    caller owns.  No entry point allocates, frees or synchronises anything:
 *    every call validates on the host, enqueues its kernels and returns.
 *  - Workspace.  A GEMM launch whose K is split over several workgroups
 *    exchanges row statistics and partial sums through a caller-owned device
 *    buffer `workspace` of `workspace_bytes` bytes; sk_gemm_workspace_size
 *    gives the bytes a call needs (0 for most calls: then `workspace` may be
 *    NULL).  The buffer must be 256-byte aligned and its contents must be zero
 *    before the first call that uses it (e.g. one hipMemset after
 *    allocation); each launch leaves it ready for the next, whatever the
 *    shapes of the calls that share it.  Calls that share one workspace must
 *    be ordered (one stream, or events); calls with different workspaces may
 *    run concurrently on different streams.  A missing, misaligned or too
 *    small workspace is SK_ERR_WORKSPACE.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work and return; nothing synchronises the host.
 *  - Validation is synchronous and happens before any GPU work: on any status
 *    other than SK_OK nothing was launched and no memory was touched.
 *    A device fault inside a launched kernel shows up at the caller's next
 *    synchronisation, not in the return value.
 *  - There is no silent fallback: a shape this backend does not handle
 *    returns SK_ERR_UNSUPPORTED rather than running a slower path.
 *  - NaN/Inf inputs are outside the contract.
 */
#ifndef SK_REPACK_H
#define SK_REPACK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SK_OK = 0,
    SK_ERR_NULL = 1,        /* a required pointer is NULL                                   */
    SK_ERR_SHAPE = 2,       /* the format's shape rules [FMT] fail, or M not in 1..8, N < 1,
                               ld < K, or `bytes` does not match N, K, G                    */
    SK_ERR_ALIGN = 3,       /* a pointer (or a row stride in bytes) is not 16-byte aligned  */
    SK_ERR_FORMAT = 4,      /* wrong entry point for the weight's format, unknown format or
                               dtype, or the codebook is missing / given when not allowed    */
    SK_ERR_LAYOUT = 5,      /* GEMM on a canonical (not repacked) weight, repack of an
                               already repacked weight, or unrepack of a canonical one      */
    SK_ERR_HIP = 6,         /* a HIP runtime call failed (launch error, no device, ...)    */
    SK_ERR_UNSUPPORTED = 7, /* allowed by [FMT] but not by this backend (see below)         */
    SK_ERR_WORKSPACE = 8    /* the call needs a workspace and `workspace` is NULL, not
                               256-byte aligned, or smaller than sk_gemm_workspace_size   */
} sk_status;

typedef enum { SK_F32 = 0, SK_BF16 = 1 } sk_dtype;

typedef enum {
    SK_W4_SYM = 0,          /* 4-bit two's-complement weights, FP32 group scales [FMT]     */
    SK_W4_CODEBOOK = 1,     /* 4-bit unsigned index into a float[16] table [FMT]           */
    SK_W6_SYM = 2           /* 6-bit two's-complement weights, FP32 group scales [FMT]     */
} sk_format;

typedef enum {
    SK_LAYOUT_CANONICAL = 0,  /* the storage layout below                                  */
    SK_LAYOUT_STREAM = 1      /* the library's interleaved stream layout (opaque)           */
} sk_layout;

/*
 * Weight descriptor.  The struct lives in host memory and is owned by the
 * caller; `data` and `codebook` are device pointers, also caller-owned.
 *
 * Canonical layout of `data` (SK_LAYOUT_CANONICAL), one allocation of
 * `bytes` = N*K*bits/8 + N*(K/G)*4 bytes:
 *   packed weights, [N][K*bits/8] uint8, row-major:
 *     W4 / codebook: byte j of a row holds element 2j in the low nibble and
 *       2j+1 in the high nibble (W4: two's complement in [-8,7]; codebook:
 *       unsigned index in [0,15]);
 *     W6: every 3 bytes are a little-endian 24-bit word with 4 consecutive
 *       elements, element r at bits 6r..6r+5, two's complement in [-32,31];
 *   followed directly by the scales, [N][K/G] float32, row-major; group j of
 *   row n covers k = j*G .. j*G+G-1 (no zero point: weights are symmetric).
 * After sk_repack_w4a8 the same bytes hold the stream layout; only this
 * library reads it.  `bytes` never changes.
 */
typedef struct {
    int32_t n;                /* N: output features                                        */
    int32_t k;                /* K: input features                                         */
    int32_t group;            /* G: group size along K                                     */
    int32_t format;           /* sk_format                                                 */
    int32_t layout;           /* sk_layout; set by sk_repack_w4a8 / sk_unrepack_w4a8       */
    int32_t reserved;         /* must be 0                                                 */
    void*   data;             /* device, 16-byte aligned                                   */
    size_t  bytes;            /* N*K*bits/8 + N*(K/G)*4                                    */
    const float* codebook;    /* device float[16] for SK_W4_CODEBOOK, else NULL            */
} sk_weight;

/*
 * Backend restrictions (returned as SK_ERR_UNSUPPORTED; [FMT] allows
 * accelerated backends to add shape limits):
 *   K % 128 == 0; G in {32, 64, 128} for SK_W4_SYM and SK_W6_SYM and
 *   G in {16, 32, 64, 128} for SK_W4_CODEBOOK; N <= 2^24;
 *   16 rows of one weight (16*K*bits/8 + 16*(K/G)*4 bytes) <= 256 KiB;
 *   K <= 17408 for the GEMM entry points.
 */

/* Human-readable name of a status code (static string, never NULL; any other
 * integer gives "unknown status"). */
const char* sk_status_string(sk_status s);

/*
 * One-time, in-place repack [LIN]: rewrites `w->data` from the canonical
 * layout into the stream layout, in which every 16-row tile's weights and
 * their group scales sit together in the order the GEMM workgroups consume
 * them.  Every format is accepted (the name follows the W4A8 case).
 * No device memory is allocated: the permutation is done with in-place
 * rotations and an in-register per-tile reorder.  Weight codes keep their
 * two's-complement values; only their positions change.
 * On success sets w->layout = SK_LAYOUT_STREAM (the host struct is updated at
 * enqueue time; the bytes are ready when the stream reaches this point).
 * Errors: NULL, SHAPE, ALIGN, FORMAT, LAYOUT (already repacked), UNSUPPORTED, HIP.
 */
sk_status sk_repack_w4a8(sk_weight* w, void* stream);

/*
 * Inverse of sk_repack_w4a8, in place: restores the canonical bytes exactly
 * and sets w->layout = SK_LAYOUT_CANONICAL.  For saving a loaded model and for
 * tests.  Errors as sk_repack_w4a8 (LAYOUT if the weight is canonical).
 */
sk_status sk_unrepack_w4a8(sk_weight* w, void* stream);

/*
 * Bytes of workspace a GEMM call needs: a call of any GEMM entry point with a
 * weight of n x k, group size `group`, format `format`, M = m rows and
 * `prologue` (0 none, 1 RMSNorm, 2 SwiGLU; the split-path entry points use 0;
 * for sk_gemm_experts, n = n_list * rows_per_expert).  *bytes = 0 when the
 * call needs none.  The size depends on the device the call runs on (its
 * compute-unit count): query with that device current.  It is 16 KiB plus
 * 128 * M * S bytes per 16-row tile, S being the number of K-slices the
 * launch uses (at most 32).
 * Errors: NULL, FORMAT, SHAPE, UNSUPPORTED (as for the GEMM calls).
 */
sk_status sk_gemm_workspace_size(int n, int k, int group, int format, int m, int prologue,
                                 size_t* bytes);

/*
 * Skinny W4A8 linear [LIN]: y[M][N] = sx[m] * sum_j s[n][j] * P[m][n][j],
 * P = per-group integer dot product of the weights (or, for the codebook,
 * the float levels) with q, where (q, sx) = per-row int8 quantisation of x
 * (sx = absmax/127, q = round-half-even(x/sx) clamped to +-127, all-zero row
 * -> sx = 0), done inside the launch [FMT activations].
 * Codebook: each level enters as the sum of two bf16 values (hi + lo, within
 * 2^-17 of the float level) multiplied by q exactly and summed in fp32, so P
 * is a float close to sum(level * q) rather than an exact integer.
 *   w  : repacked SK_W4_SYM or SK_W4_CODEBOOK weight
 *   x  : device [M][K], row-major, dtype xt (SK_F32 or SK_BF16), 16-byte aligned
 *   m  : 1..8
 *   y  : device [M][N] float32, row-major, 16-byte aligned (fully overwritten)
 *   workspace, workspace_bytes : see the conventions above
 * Errors: NULL, SHAPE, ALIGN, FORMAT (not a W4 format), LAYOUT, UNSUPPORTED,
 *         WORKSPACE, HIP.
 */
sk_status sk_gemm_w4a8(const sk_weight* w, const void* x, int xt, int m,
                       float* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sk_gemm_w4a8 for callers that cannot allocate or pass device memory (code
 * under stream capture that must not reach the allocator, tight serving
 * loops, harnesses that forbid allocation): the same checks, kernels and
 * results, with the workspace replaced by a fixed scratch array in the
 * library's device memory (4 MiB per device, held by each GPU the library
 * runs on until the process ends).  Calls that would need a larger workspace
 * return SK_ERR_WORKSPACE.  The first call on a device also enqueues a clear
 * of that device's scratch on `stream` (a kernel launch).  All calls of this
 * entry point on one device share its scratch: calls that overlap in time on
 * one GPU race and must be ordered (one stream, or events).
 * Errors: as sk_gemm_w4a8.
 */
sk_status sk_gemm_w4a8_noalloc(const sk_weight* w, const void* x, int xt, int m,
                               float* y, void* stream);

/* Same for a repacked SK_W6_SYM weight [LIN] [FMT]. */
sk_status sk_gemm_w6a8(const sk_weight* w, const void* x, int xt, int m,
                       float* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * RMSNorm prologue fused into the quantisation [LIN]:
 *   h[m][k] = fp32(fp32(x[m][k] * r[m]) * gamma[k]),
 *   r[m] = fp32(1 / fp32(sqrt(fp32(fp32(ss[m]/K) + eps)))),
 *   ss[m] = sum_k x[m][k]^2 in float64,
 * then y = linear(w, h) exactly as sk_gemm_w4a8 / sk_gemm_w6a8 would with x = h.
 * h never leaves registers/LDS.  Any weight format.
 *   gamma: device [K] float32, 16-byte aligned.  eps: added in fp32.
 */
sk_status sk_gemm_fused_rmsnorm(const sk_weight* w, const void* x, int xt,
                                const float* gamma, float eps, int m,
                                float* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * SwiGLU prologue fused into the quantisation [LIN]:
 *   h[m][k] = fp32(fp32(g / fp32(1 + E(-g))) * u),  g = gate[m][k], u = up[m][k],
 * where E is a fixed float32 exp (Cody-Waite reduction by ln 2 in two parts,
 * degree-7 Taylor polynomial in Horner form, scaling by 2^n in two exact
 * steps; arguments >= 89 give +inf, <= -104 give 0), then y = linear(w, h).
 *   gate, up: device, rows of K elements with row stride `ld` elements
 *             (ld >= K; ld * element size a multiple of 16 bytes), dtype xt.
 * Any weight format.
 */
sk_status sk_gemm_fused_swiglu(const sk_weight* w, const void* gate, const void* up,
                               int64_t ld, int xt, int m, float* y, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Expert bank [FMT, embeddings and MoE: grouped W4A8/W6A8 banks store their
 * experts' output rows flattened to E * N]: `bank` is one repacked weight of
 * E * rows_per_expert rows (any format), expert e owning rows
 * [e * rows_per_expert, (e + 1) * rows_per_expert).  One launch computes, for
 * each of the n_list listed experts, its rows times x (quantised once):
 *   y[m][i * rows_per_expert + j] = (expert experts[i], row j) . x[m]
 *   experts : DEVICE array of n_list int32 expert ids (4-byte aligned), read
 *             by the kernel when it runs, so a captured graph replays with
 *             whatever ids the array then holds (e.g. a router's output).
 *             Repeats are allowed.  An id outside [0, E) cannot be rejected on
 *             the host: that expert's block of y is written as NaN (no memory
 *             outside the bank is read).
 *   y       : device [M][n_list * rows_per_expert] float32, 16-byte aligned
 *   rows_per_expert a multiple of 16 dividing bank->n; n_list >= 1 and
 *   n_list * rows_per_expert <= 2^24.
 * Each listed expert's output is what sk_gemm_w4a8 / sk_gemm_w6a8 gives on
 * that expert's rows alone: the same q and the same int32 partials; only the
 * grouping of the fp32 sums across waves may differ with the launch plan.
 * Errors: NULL, SHAPE (rows_per_expert, n_list), ALIGN, FORMAT, LAYOUT,
 * UNSUPPORTED, WORKSPACE, HIP.
 */
sk_status sk_gemm_experts(const sk_weight* bank, int rows_per_expert, const int32_t* experts,
                          int n_list, const void* x, int xt, int m, float* y, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * The split path, kept to measure what the stream layout and the fused
 * quantisation buy [LIN]: the pages' earlier design read the weights and
 * their scales from two separate tensors and quantised the activations in a
 * launch of its own, with q going through memory.  Here the weight stays in
 * the canonical layout (codes region, then scales region), and the
 * quantisation can run as its own launch.  Results equal those of the fused
 * entry points bit for bit (same q, same partial sums in the same order).
 */

/*
 * Per-row int8 quantisation as its own launch: q[m][k] and sx[m] exactly as
 * sk_gemm_w4a8 computes them inside its launch [FMT activations].
 *   x  : device [M][K] row-major, dtype xt, 16-byte aligned
 *   q  : device [M][K] int8, 16-byte aligned (fully overwritten)
 *   sx : device [M] float32, 4-byte aligned (fully overwritten)
 *   m 1..8, K a positive multiple of 16.
 * Errors: NULL, SHAPE, ALIGN, FORMAT (dtype), HIP.
 */
sk_status sk_quantize_rows(const void* x, int xt, int m, int k, int8_t* q, float* sx,
                           void* stream);

/*
 * The prologues as launches of their own, for the split path: h (device
 * [M][K] float32, rows K apart, 16-byte aligned) is written to memory with
 * the fused entry points' arithmetic, so sk_gemm_w4a8(w, h) or
 * sk_quantize_rows(h) then sees the h the fused call keeps on chip [LIN].
 *   sk_prologue_rmsnorm: h = RMSNorm(x) exactly as sk_gemm_fused_rmsnorm;
 *     x [M][K] of dtype xt, gamma [K] float32, both 16-byte aligned.
 *   sk_prologue_swiglu: h = SwiGLU(gate, up) exactly as sk_gemm_fused_swiglu;
 *     gate, up rows of K elements with row stride `ld` elements (ld >= K,
 *     ld * element size a multiple of 16 bytes), dtype xt, 16-byte aligned.
 *   m 1..8, K a positive multiple of 16.
 * Errors: NULL, SHAPE, ALIGN, FORMAT (dtype), HIP.
 */
sk_status sk_prologue_rmsnorm(const void* x, int xt, const float* gamma, float eps, int m, int k,
                              float* h, void* stream);
sk_status sk_prologue_swiglu(const void* gate, const void* up, int64_t ld, int xt, int m, int k,
                             float* h, void* stream);

/*
 * sk_gemm_w4a8 on a weight left in the canonical layout
 * (w->layout == SK_LAYOUT_CANONICAL, no repack): the workgroups read each
 * tile's codes and its scales from the two regions.  SK_W4_SYM only; the
 * backend restrictions of sk_gemm_w4a8 apply.
 * Errors: as sk_gemm_w4a8 (LAYOUT if the weight is repacked, FORMAT if it is
 * not SK_W4_SYM).
 */
sk_status sk_gemm_w4a8_canonical(const sk_weight* w, const void* x, int xt, int m,
                                 float* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same GEMM with the activations already quantised (by sk_quantize_rows):
 *   q  : device [M][K] int8, 16-byte aligned;  sx : device [M] float32, 4-byte aligned.
 * Errors: as sk_gemm_w4a8_canonical.
 */
sk_status sk_gemm_w4a8_canonical_q(const sk_weight* w, const int8_t* q, const float* sx, int m,
                                   float* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test hook: the GEMM kernels instantiated with an export flag.  Runs the same
 * computation as the entry point selected by `prologue` (0 = none,
 * 1 = RMSNorm, 2 = SwiGLU; `x2`, `ld`, `gamma`, `eps` as there; for prologue 0
 * and 1 `ld` is ignored and rows are K apart) and additionally writes
 *   q_out  [M][K]     int8    : the quantised activations the kernel used,
 *   sx_out [M]        float32 : their scales,
 *   p_out  [M][N][K/G] int32  : the per-group integer partials (integer
 *                               formats; must be NULL for the codebook).
 * Any of q_out / sx_out / p_out may be NULL.  p_out is zeroed by the call.
 */
sk_status sk_debug_gemm(const sk_weight* w, int prologue, const void* x, const void* x2,
                        int64_t ld, int xt, const float* gamma, float eps, int m,
                        float* y, int8_t* q_out, float* sx_out, int32_t* p_out,
                        void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SK_REPACK_H */
