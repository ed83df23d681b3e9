/*
 * sk_attention.h -- C ABI of the grouped-query decode attention in the same
 * library (libsk_repack.so); status codes are those of sk_repack.h.
 *
 *   O[m, h, :] = softmax_j( scale * <q[m, h], K[h/G, j]> ) . V[h/G, j, :],
 *                j = 0 .. L - M + m,   m < M <= 8,  G = Hq / Hkv,
 *
 * Source, cited by page title and section:
 *  [ATT]  "在 ComfyUI 中将 LLM token 速率翻倍" (Doubling the LLM token rate in
 *         ComfyUI), section "关注 attention!": every fourth layer of the
 *         hybrid model is grouped-query attention with a KV cache; its decode
 *         kernel takes one token, or a few MTP draft rows with causal
 *         verification, without building a mask; it splits the cached prefix
 *         over many workgroups so that a tiny query still fills the GPU, and
 *         the last workgroup to finish merges the partial results inside the
 *         same launch.
 *
 * Readings where [ATT] is silent:
 *  - The M query rows are the last M positions of the sequence and their keys
 *    and values are already in the cache (L entries), so row m sees entries
 *    0 .. L - M + m (a causal mask aligned to the bottom-right corner).
 *  - Query head h reads KV head h / G (consecutive query heads share a KV head).
 *  - Head dimension 128; q, K and V are bfloat16; O is float32.
 *
 * KV cache layout (this library's; every entry point below uses it).  One
 * device buffer of Hkv * (cap/32) * 16384 bytes; head hk, block b (cache
 * entries 32b .. 32b+31) starts at byte ((hk * cap/32) + b) * 16384:
 *   bytes [0, 8192)      K: 8 tiles of 1 KiB, tile i = 4*kh + c; in tile i,
 *                        bytes 16*l .. 16*l+15 (l = 0..63) hold the 8 bf16
 *                        K[32b + 16*kh + (l % 16)][32*c + 8*(l / 16) + e],
 *                        e = 0..7;
 *   bytes [8192, 16384)  V: 8 tiles of 1 KiB, tile t covers dimensions
 *                        16t .. 16t+15; bytes 16*l + 2*e hold
 *                        V[32b + key(l / 16, e)][16*t + (l % 16)], where
 *                        key(g, e) = 4g + e for e < 4 and 16 + 4g + (e - 4)
 *                        for e >= 4.
 * Each tile is exactly the operand of one 64-lane matrix instruction, so a
 * block is one contiguous 16 KiB read.  Entries at or beyond L are never read
 * into the result (their contents do not matter).
 *
 * Conventions: pointers are DEVICE pointers to caller-owned memory unless
 * stated; `stream` is a hipStream_t as void*; validation is synchronous and a
 * rejected call launches nothing.  Nothing here allocates, frees or
 * synchronises.  A launch that splits the prefix over several ranges per KV
 * head exchanges partial results through a caller-owned device `workspace`
 * (same rules as the GEMM workspace of sk_repack.h: 256-byte aligned, zero
 * before its first use, left ready for the next call of any shape; calls
 * sharing one workspace must be ordered): a generation word, one arrival
 * counter per KV head and one flag per (KV head, prefix range), 133376 bytes
 * in all, then Hkv * ranges * 16*ceil(M*G/16) * 130 floats of partial
 * results (at most 64 ranges per head).  sk_attention_workspace_size gives the
 * bytes a call needs (0 when the prefix is not split).
 */
#ifndef SK_ATTENTION_H
#define SK_ATTENTION_H

#include <stdint.h>

#include "sk_repack.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Writes t new entries (positions pos .. pos+t-1) of every KV head into the
 * cache [ATT: the KV cache of the grouped-query layer].
 *   kv      cache buffer in the layout above, Hkv * cap/32 * 16384 bytes
 *   cap     cache capacity in entries, a multiple of 32
 *   k_new, v_new   [t][Hkv][128] bf16 (uint16 bits), 16-byte aligned
 * Errors: NULL, SHAPE (hkv < 1, t < 1, pos < 0, pos + t > cap, cap % 32),
 *         ALIGN, HIP.
 */
sk_status sk_kv_append(void* kv, int hkv, int cap, int pos, int t,
                       const uint16_t* k_new, const uint16_t* v_new, void* stream);

/*
 * Decode attention [ATT] for M query rows against the first L cache entries.
 *   q       [M][Hq][128] bf16 (uint16 bits), 16-byte aligned
 *   kv      cache (layout above) of capacity cap entries, L <= cap
 *   scale   softmax scale (1/sqrt(128) for the usual attention)
 *   out     [M][Hq][128] float32, 16-byte aligned
 * The prefix is split into ranges of 32-entry blocks over many workgroups
 * (one per range and KV head); each publishes its partial result, and the
 * last workgroup of each KV head to start combines the ranges' results
 * (log-sum-exp rescaling, fixed range order) and writes out, in the same
 * launch.
 * Errors: NULL, SHAPE (M not in 1..8, hq % hkv, L < M, L > cap, cap % 32,
 *         scale not finite and > 0), UNSUPPORTED (M * Hq / Hkv > 64,
 *         Hkv > 512, cap > 4194304), ALIGN, WORKSPACE, HIP.
 */
sk_status sk_decode_attention(const uint16_t* q, int m, int hq, int hkv,
                              const void* kv, int cap, int len, float scale,
                              float* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Bytes of workspace sk_decode_attention needs for these sizes on the current
 * device (0 when the prefix is not split).
 * Errors: NULL, SHAPE, UNSUPPORTED (as sk_decode_attention), HIP (no device).
 */
sk_status sk_attention_workspace_size(int m, int hq, int hkv, int len, size_t* bytes);

/*
 * Host-side packing into the cache layout (no GPU): k and v are host arrays
 * [Hkv][len][128] bf16; out is a host buffer of Hkv * cap/32 * 16384 bytes;
 * entries len .. cap-1 are zero-filled.  For building a cache on the host
 * and for tests.  Errors: NULL, SHAPE.
 */
sk_status sk_kv_pack_host(const uint16_t* k, const uint16_t* v, int hkv, int len, int cap,
                          void* out);

/*
 * Planning and tuning hooks (host only).
 * sk_test_attention_plan: the split the next sk_decode_attention with these
 *   sizes would use: *splits ranges of *blocks_per_split 32-entry blocks per
 *   KV head (one workgroup each), for a device with `cus` compute units
 *   (0 = the current device's count).
 * sk_test_set_attention_split: force blocks per split (0 = planner).
 */
sk_status sk_test_attention_plan(int m, int hq, int hkv, int len, int cus, int* splits,
                                 int* blocks_per_split);
sk_status sk_test_set_attention_split(int blocks_per_split);

#ifdef __cplusplus
}
#endif

#endif /* SK_ATTENTION_H */
