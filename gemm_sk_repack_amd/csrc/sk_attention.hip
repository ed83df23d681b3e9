// sk_attention.hip -- grouped-query decode attention over a tiled KV cache
// for gfx950 (MI355X), plus the cache's append and host packing.
//
// ("Doubling the LLM token rate in ComfyUI", section on attention: a decode
// kernel for one token or a few MTP draft rows with causal verification, no
// materialised mask, the cached prefix split over many workgroups and the
// partial results merged by the last workgroup in the same launch.)
//
// Launch: one 256-thread workgroup per (prefix range s, KV head hk).  The
// G query heads that share KV head hk and the M verification rows form
// R = M*G query rows, handled together so that every K/V byte is read once.
// Each wave takes every fourth 32-entry block of the range and keeps an
// online-softmax state (running max in log2 units, running sum, unnormalised
// output) in registers:
//
//   S^T = K . Q^T        v_mfma_f32_16x16x32_bf16, K tile = A operand (16
//                        entries x 32 dims per instruction), the query rows
//                        = B operand (16 rows per query tile);
//   causal limit         entry j is kept for row (m, .) iff j <= L - M + m,
//                        by a compare per score (no mask tensor);
//   P = exp2(S*scale*log2e - max)   fp32, then split P = hi + lo, each
//                        bfloat16 (round to nearest even), so that the
//                        product with bfloat16 V keeps ~16 bits of P;
//   O^T += V^T . P^T     the V tile = A operand, hi and lo = B operands.
//
// The score accumulator's lane layout (lane l holds query row l%16 and entries
// 4*(l/16)+v) is exactly the B-operand layout of the second product, so P
// never moves between lanes; the cache layout puts V's entries in that order.
// The four waves' states are combined through LDS in wave order.  With one
// range the workgroup writes O.  Otherwise every workgroup counts itself on
// its head's arrival counter when it starts, stores its partial state
// write-through and publishes it by a release store of the launch's tag
// (a generation number kept in the workspace) into its flag; the head's
// last workgroup to start waits for all flags (acquire), combines the ranges
// in range order and writes O, inside the same launch.  Results do not
// depend on timing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/sk_attention.h"

#define SK_EXPORT extern "C" __attribute__((visibility("default")))

namespace ska {

constexpr int HD = 128;                       // head dimension
constexpr int BK = 32;                        // cache entries per block
constexpr int BLOCK_BYTES = 2 * BK * HD * 2;  // K tile + V tile, bf16
constexpr int AW = 4;                         // waves per workgroup
constexpr int AT = AW * 64;
constexpr int kMaxRows = 64;                  // M * G
constexpr int kMaxSplits = 64;
constexpr int kMaxKvHeads = 512;              // keeps the partial states under 2 GiB
constexpr int kMaxEntries = 1 << 22;          // keeps one range under 2 GiB
constexpr int kSpin = 1 << 20;                // polls of a flag before giving up (NaN)
constexpr int PSTRIDE = HD + 2;               // floats per partial query row: O[128], max, sum
constexpr int kSC1 = 16;                      // cache policy: system-coherent (write-through) access
constexpr int kNT = 2;                        // cache policy: non-temporal (the cache is read once per call)
constexpr int kOutside = 0x7FFFFFF0;          // a buffer offset past any workspace: reads zero

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

struct AttnArgs {
    const uint16_t* q;   // [M][Hq][128]
    const uint8_t* kv;   // cache, layout in sk_attention.h
    float* out;          // [M][Hq][128]
    float* part;         // partial states: [Hkv][nsplit]{ O [RP][128], (max, sum) [RP][2] }
    uint32_t* flag;      // [Hkv][nsplit] partial state published (the launch's tag)
    uint32_t* hdr;       // [0] generation of the last multi-range launch, [1] workgroups done
    uint32_t* cnt;       // [Hkv] arrivals
    int m, hq, g, r, len, nbc, nblk, bps, nsplit, nwg, part_bytes;
    float sl2;           // scale * log2(e)
};

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline uint32_t peek_gen(const uint32_t* hdr) {
    return __hip_atomic_load(hdr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes a partial state.  Its data was stored write-through (sc1) and the
// barrier before the call ordered every thread's stores before this one; the
// release store then makes them visible at device scope before the flag
// shows the launch's tag.
__device__ inline void publish(uint32_t* flag, uint32_t tag) {
    __hip_atomic_store(flag, tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls a flag until it shows `tag`; the caller issues one acquire fence after
// all its flags are seen.  The bound only guards against a hang (false then;
// the caller writes NaN).
__device__ inline bool await_flag(const uint32_t* flag, uint32_t tag) {
    for (int it = 0; it < kSpin; ++it)
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag) return true;
    return false;
}

// Write-through 16-byte store into the workspace (offset in bytes from its base).
__device__ inline void wt_store(const __amdgpu_buffer_rsrc_t& ws, int off, float4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), ws, off, 0, kSC1);
}

template <int NQT>
__global__ __launch_bounds__(AT) void attn_kernel(AttnArgs a) {
    constexpr int RP = NQT * 16;              // query rows padded to whole tiles
    constexpr int NSLOT = 2;                  // blocks held in registers (more measured slower)
    // dynamic LDS (smem below): the waves' states, [AW][NQT][34][64] floats,
    // later reused by the merges
    static_assert(AW * NQT * 34 * 64 >= 2 * kMaxSplits * RP, "merge scratch");
    __shared__ float den[RP], dmx[RP];        // staging of a range's (max, sum) per row
    __shared__ int last;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int s = blockIdx.x, hk = blockIdx.y;
    const int M = a.m, G = a.g, R = a.r, L = a.len;
    // this launch's tag: one more than the previous multi-range launch's.  The
    // generation word and the done counter share a cache line and thread 0
    // reads the one before it counts itself on the other, so every workgroup
    // has read the generation before the last one to count replaces it.
    const uint32_t tag = a.nsplit > 1 ? peek_gen(a.hdr) + 1u : 0u;
    // With several ranges, count this workgroup on its head's counter right
    // away: the last to start merges, after its own loop, waiting for the
    // others' published partial states.  Counting early keeps the atomics'
    // round trip off the end of the launch.
    uint32_t arrived = 0, done = 0;
    if (a.nsplit > 1 && tid == 0) {
        arrived = __hip_atomic_fetch_add(&a.cnt[hk], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        done = __hip_atomic_fetch_add(&a.hdr[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // 1. this lane's query rows (B operand: row t*16 + l16, dims 32c + 8*g4 + e)
    uint4 qv[NQT][4];
    int lim[NQT];
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        const int r = t * 16 + l16;
        if (r < R) {
            const int mm = r / G, hg = r - mm * G;
            const uint4* qp = reinterpret_cast<const uint4*>(a.q + (size_t)(mm * a.hq + hk * G + hg) * HD);
#pragma unroll
            for (int c = 0; c < 4; ++c) qv[t][c] = qp[c * 4 + g4];
            lim[t] = L - M + mm;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) qv[t][c] = make_uint4(0u, 0u, 0u, 0u);
            lim[t] = L - 1;                   // padding rows: zero queries, never all masked
        }
    }

    // 2. this wave's blocks: b0 + wv, b0 + wv + 4, ... below b1.  The main
    //    loop takes the range's whole blocks (below nfull = L / 32) through a
    //    buffer resource covering exactly them, so the pipeline's look-ahead
    //    loads past them return zeros without touching memory and every wave
    //    issues the same, static load pattern; a final partial block is done
    //    after the loop by the wave that owns it.
    const int wu = __builtin_amdgcn_readfirstlane(wv);
    const int b0 = s * a.bps;
    const int b1 = min(b0 + a.bps, a.nblk);
    const int bfull = min(b1, L / BK);
    const int nw = (bfull - b0 > wu) ? (bfull - b0 - wu + AW - 1) / AW : 0;
    uint8_t* const rbase = const_cast<uint8_t*>(a.kv + ((size_t)hk * a.nbc + b0) * BLOCK_BYTES);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(rbase, (short)0, max(bfull - b0, 0) * BLOCK_BYTES, 0x00020000);

    float mrun[NQT], lrun[NQT];
    v4f o[NQT][8];
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        mrun[t] = -INFINITY;
        lrun[t] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    auto load = [&](uint4 (&kb)[8], uint4 (&vb)[8], const __amdgpu_buffer_rsrc_t& rs, int i) {
        const int off = (wu + AW * i) * BLOCK_BYTES + lane * 16;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            kb[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + j * 1024, 0, kNT));
#pragma unroll
        for (int j = 0; j < 8; ++j)
            vb[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 8192 + j * 1024, 0, kNT));
    };

    // Max over the four lanes of a query row (lanes l, l^16, l^32, l^48).
    auto rowmax = [](float v) {
        const auto a16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(a16[0]), __uint_as_float(a16[1]));
        const auto a32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return fmaxf(__uint_as_float(a32[0]), __uint_as_float(a32[1]));
    };

    // One block: i-th of this wave; `ok` false makes every score -inf (a
    // look-ahead slot past the range, whose K and V read as zeros).
    auto compute = [&](const uint4 (&kb)[8], const uint4 (&vb)[8], int i, bool ok) {
        const int key0 = (b0 + wu + AW * i) * BK + 4 * g4;
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
            v4f s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb[c]), as_bf16x8(qv[t][c]), s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb[4 + c]), as_bf16x8(qv[t][c]), s1, 0, 0, 0);
            }
            float x[8];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                x[v] = (ok && key0 + v <= lim[t]) ? s0[v] * a.sl2 : -INFINITY;
                x[4 + v] = (ok && key0 + 16 + v <= lim[t]) ? s1[v] * a.sl2 : -INFINITY;
            }
            const float mx = rowmax(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                          fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
            const float mnew = fmaxf(mrun[t], mx);
            const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(mrun[t] - mu);
            mrun[t] = mnew;
            // P = hi + lo, both bf16 (round to nearest even): hi = bf16(p),
            // lo = bf16(p - hi), where p - hi is exact in fp32
            uint32_t ph2[4], pl2[4];
            float ps = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float p0 = __builtin_amdgcn_exp2f(x[2 * j] - mu);
                const float p1 = __builtin_amdgcn_exp2f(x[2 * j + 1] - mu);
                ps += p0;
                ps += p1;
                const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
                const float r0 = p0 - __uint_as_float(h << 16);
                const float r1 = p1 - __uint_as_float(h & 0xFFFF0000u);
                ph2[j] = h;
                pl2[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){r0, r1}, bf16x2));
            }
            lrun[t] = lrun[t] * alpha + ps;
            const uint4 ph = make_uint4(ph2[0], ph2[1], ph2[2], ph2[3]);
            const uint4 pl = make_uint4(pl2[0], pl2[1], pl2[2], pl2[3]);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                o[t][dt] *= alpha;
                o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vb[dt]), as_bf16x8(ph), o[t][dt], 0, 0, 0);
                o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vb[dt]), as_bf16x8(pl), o[t][dt], 0, 0, 0);
            }
        }
    };

    // 3. the wave's blocks through NSLOT register slots: while a block is
    //    computed, the next NSLOT-1 blocks' loads are in flight.  The body is
    //    branch-free so that consecutive blocks' instructions interleave.
    if (nw > 0) {
        uint4 kb[NSLOT][8], vb[NSLOT][8];
#pragma unroll
        for (int u = 0; u < NSLOT; ++u) load(kb[u], vb[u], rsrc, u);
        for (int i = 0; i < nw; i += NSLOT) {
#pragma unroll
            for (int u = 0; u < NSLOT; ++u) {
                compute(kb[u], vb[u], i + u, i + u < nw);
                load(kb[u], vb[u], rsrc, i + u + NSLOT);
            }
        }
    }
    // the prefix's final partial block, if this range holds it: entries at or
    // past L may hold anything (0 * Inf would be NaN), so their V values are
    // zeroed before the product
    if (bfull < b1 && ((bfull - b0) & (AW - 1)) == wu) {
        const int it = (bfull - b0) / AW;          // this wave's index of the block
        const __amdgpu_buffer_rsrc_t rt =
            __builtin_amdgcn_make_buffer_rsrc(rbase, (short)0, (b1 - b0) * BLOCK_BYTES, 0x00020000);
        uint4 kb[8], vb[8];
        load(kb, vb, rt, it);
        const int nv = L - bfull * BK;             // valid entries, 1..31
        uint32_t km[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e0 = 2 * j, e1 = 2 * j + 1;
            const int k0 = e0 < 4 ? 4 * g4 + e0 : 16 + 4 * g4 + e0 - 4;
            const int k1 = e1 < 4 ? 4 * g4 + e1 : 16 + 4 * g4 + e1 - 4;
            km[j] = (k0 < nv ? 0x0000FFFFu : 0u) | (k1 < nv ? 0xFFFF0000u : 0u);
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            vb[dt].x &= km[0];
            vb[dt].y &= km[1];
            vb[dt].z &= km[2];
            vb[dt].w &= km[3];
        }
        compute(kb, vb, it, true);
    }
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        const auto a16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lrun[t]), __float_as_uint(lrun[t]), false, false);
        const float l2 = __uint_as_float(a16[0]) + __uint_as_float(a16[1]);
        const auto a32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l2), __float_as_uint(l2), false, false);
        lrun[t] = __uint_as_float(a32[0]) + __uint_as_float(a32[1]);
    }

    // 4. combine the four waves' states: every wave parks its state in LDS,
    //    then each thread combines 8 of its lane's 32 output values over the
    //    waves (wave w takes values 8w .. 8w+7: dims 16*(2w + k/4) + 4*g4 + k%4,
    //    k = 0..7), always in wave order
    extern __shared__ float smem[];
    constexpr int SW = 34 * 64;               // floats per (wave, query tile) state
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        float* st = smem + (wv * NQT + t) * SW + lane;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v) st[(dt * 4 + v) * 64] = o[t][dt][v];
        st[32 * 64] = mrun[t];
        st[33 * 64] = lrun[t];
    }
    if (a.nsplit > 1 && tid == 0) {
        const int lst = arrived == (uint32_t)(a.nsplit - 1);
        if (lst) __hip_atomic_store(&a.cnt[hk], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = lst;
        // generation bookkeeping: after every workgroup of the launch has read
        // the generation (each did so before counting itself), the last one
        // publishes this launch's tag for the next launch
        if (done == (uint32_t)(a.nwg - 1)) {
            __hip_atomic_store(&a.hdr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.hdr[0], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    float cm[NQT], cl[NQT], cv[NQT][8];
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        float mw[AW], ww[AW];
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < AW; ++w) {
            mw[w] = smem[(w * NQT + t) * SW + 32 * 64 + lane];
            mx = fmaxf(mx, mw[w]);
        }
        const float mu = (mx == -INFINITY) ? 0.0f : mx;
        float l = 0.0f;
#pragma unroll
        for (int w = 0; w < AW; ++w) {
            ww[w] = __builtin_amdgcn_exp2f(mw[w] - mu);
            l = __builtin_fmaf(smem[(w * NQT + t) * SW + 33 * 64 + lane], ww[w], l);
        }
        cm[t] = mx;
        cl[t] = l;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float acc = 0.0f;
#pragma unroll
            for (int w = 0; w < AW; ++w) acc = __builtin_fmaf(smem[(w * NQT + t) * SW + (8 * wv + k) * 64 + lane], ww[w], acc);
            cv[t][k] = acc;
        }
    }

    // 5. one range: write O.
    if (a.nsplit == 1) {
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
            const int r = t * 16 + l16;
            if (r < R) {
                const int mm = r / G, hg = r - mm * G;
                const float inv = 1.0f / cl[t];
                float* op = a.out + (size_t)(mm * a.hq + hk * G + hg) * HD + 4 * g4 + 32 * wv;
                *reinterpret_cast<float4*>(op) =
                    make_float4(cv[t][0] * inv, cv[t][1] * inv, cv[t][2] * inv, cv[t][3] * inv);
                *reinterpret_cast<float4*>(op + 16) =
                    make_float4(cv[t][4] * inv, cv[t][5] * inv, cv[t][6] * inv, cv[t][7] * inv);
            }
        }
        return;
    }

    //    Otherwise store the partial state, O [RP][128] then (max, sum)
    //    [RP][2] per range, and publish it with the launch's tag.  Workgroups
    //    other than the head's merger are then done.
    constexpr int CH = RP * PSTRIDE;
    float* const p0 = a.part + ((size_t)hk * a.nsplit) * CH;        // [nsplit][CH]
    const __amdgpu_buffer_rsrc_t wsr = __builtin_amdgcn_make_buffer_rsrc(a.part, (short)0, a.part_bytes, 0x00020000);
    {
        const int mine = (int)((p0 - a.part) + (size_t)s * CH);         // float offset
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
            const int r = t * 16 + l16;
            if (r < R) {
                const int pp = mine + r * HD + 4 * g4 + 32 * wv;
                wt_store(wsr, 4 * pp, make_float4(cv[t][0], cv[t][1], cv[t][2], cv[t][3]));
                wt_store(wsr, 4 * (pp + 16), make_float4(cv[t][4], cv[t][5], cv[t][6], cv[t][7]));
            }
        }
        // (max, sum) of rows 2j and 2j+1 as one 16-byte store: row r's pair
        // sits in lane l16 = r of wave 0 (g4 = 0); gather it via LDS
        if (wv == 0 && g4 == 0) {
#pragma unroll
            for (int t = 0; t < NQT; ++t) {
                dmx[t * 16 + l16] = cm[t];
                den[t * 16 + l16] = cl[t];
            }
        }
    }
    __syncthreads();
    if (tid < (R + 1) / 2) {
        const int r = 2 * tid;
        const int mine = (int)((p0 - a.part) + (size_t)s * CH);
        wt_store(wsr, 4 * (mine + RP * HD + 2 * r), make_float4(dmx[r], den[r], dmx[r + 1], den[r + 1]));
    }
    __syncthreads();
    if (tid == 0) publish(&a.flag[(size_t)hk * a.nsplit + s], tag);
    if (!last) return;

    // 6. merge (the head's last workgroup to start): wait until every range's
    //    state is published, then per row the max over the ranges, weights
    //    exp2(max_q - max), and every (row, dim) as the weighted sum in range
    //    order, divided by the weighted sum of the ranges' sums.
    float* const wq = smem;                   // [n][RP] maxima (LDS reused)
    float* const lq = smem + kMaxSplits * RP; // [n][RP] sums, then weights
    __shared__ int okf;
    auto merge = [&](const float* src, const uint32_t* flags, int n) {
        if (tid == 0) okf = 1;
        __syncthreads();
        if (tid < n) {
            if (!await_flag(&flags[tid], tag)) okf = 0;
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        const float bad = okf ? 0.0f : __builtin_nanf("");
        // Each thread owns E4 float4 items (row, 4 dims).  The first batch of
        // partial outputs is loaded before the (max, sum) pass so that both
        // round trips overlap.  Wave 0 turns the (max, sum) values into
        // per-(range, row) weights in LDS, one row per lane (R <= 64; every
        // lane computes, only lanes of real rows store).
        constexpr int E4 = RP * HD / 4 / AT;
        constexpr int QB = 32 / E4;           // partials per batch: 32 float4 in flight
        float4 acc[E4], v[QB][E4];
#pragma unroll
        for (int e = 0; e < E4; ++e) acc[e] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        // Loads through the workspace's buffer resource: an item past the n
        // ranges or the R rows gets an offset beyond the resource and reads
        // zero without a memory access, so the loads need no branches.
        const int sbase = (int)(src - a.part);
        auto fetch = [&](int q0) {
#pragma unroll
            for (int u = 0; u < QB; ++u)
#pragma unroll
                for (int e = 0; e < E4; ++e) {
                    const int i4 = tid + e * AT;
                    const int off = (q0 + u < n && i4 * 4 < R * HD) ? 4 * (sbase + (q0 + u) * CH + 4 * i4) : kOutside;
                    v[u][e] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(wsr, off, 0, 0));
                }
        };
        fetch(0);
        for (int idx = tid; idx < n * R; idx += AT) {
            const int q = idx / R, r = idx - q * R;
            const float2 ml = *reinterpret_cast<const float2*>(src + (size_t)q * CH + RP * HD + 2 * r);
            wq[q * RP + r] = ml.x;
            lq[q * RP + r] = ml.y;
        }
        __syncthreads();
        if (wu == 0) {
            // 8 ranges per round, so that the LDS reads of a round are in flight
            // together
            const int r = min(lane, R - 1);
            float mx = -INFINITY;
            for (int q0 = 0; q0 < n; q0 += 8) {
                float mv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) mv[u] = (q0 + u < n) ? wq[min(q0 + u, kMaxSplits - 1) * RP + r] : -INFINITY;
#pragma unroll
                for (int u = 0; u < 8; ++u) mx = fmaxf(mx, mv[u]);
            }
            const float m0 = (mx == -INFINITY) ? 0.0f : mx;
            float d = 0.0f;
            for (int q0 = 0; q0 < n; q0 += 8) {
                float mv[8], lv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int qq = min(q0 + u, kMaxSplits - 1);
                    mv[u] = wq[qq * RP + r];
                    lv[u] = lq[qq * RP + r];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (q0 + u < n) {
                        const float w = __builtin_amdgcn_exp2f(mv[u] - m0);
                        d = __builtin_fmaf(lv[u], w, d);
                        if (lane < R) lq[(q0 + u) * RP + r] = w;   // weights replace the sums
                    }
                }
            }
            if (lane < R) den[lane] = 1.0f / (d + bad);
        }
        __syncthreads();
        for (int q0 = 0; q0 < n; q0 += QB) {
            if (q0 > 0) fetch(q0);
#pragma unroll
            for (int u = 0; u < QB; ++u)
#pragma unroll
                for (int e = 0; e < E4; ++e) {
                    // past the n ranges v is zero and the weight is zero: no branch
                    const float w = (q0 + u < n) ? lq[min(q0 + u, kMaxSplits - 1) * RP +
                                                      min((tid + e * AT) * 4 / HD, RP - 1)]
                                                 : 0.0f;
                    acc[e].x = __builtin_fmaf(v[u][e].x, w, acc[e].x);
                    acc[e].y = __builtin_fmaf(v[u][e].y, w, acc[e].y);
                    acc[e].z = __builtin_fmaf(v[u][e].z, w, acc[e].z);
                    acc[e].w = __builtin_fmaf(v[u][e].w, w, acc[e].w);
                }
        }
#pragma unroll
        for (int e = 0; e < E4; ++e) {
            const int i4 = tid + e * AT;
            if (i4 * 4 < R * HD) {
                const int r = (4 * i4) / HD, d = 4 * i4 - r * HD;
                const int mm = r / G, hg = r - mm * G;
                const float inv = den[r];
                *reinterpret_cast<float4*>(a.out + (size_t)(mm * a.hq + hk * G + hg) * HD + d) =
                    make_float4(acc[e].x * inv, acc[e].y * inv, acc[e].z * inv, acc[e].w * inv);
            }
        }
    };

    merge(p0, a.flag + (size_t)hk * a.nsplit, a.nsplit);
}

// Append t entries: one thread per (entry, head, 8 dimensions).
__global__ __launch_bounds__(256) void kv_append_kernel(uint8_t* kv, int hkv, int nbc, int pos, int t,
                                                        const uint16_t* kn, const uint16_t* vn) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= t * hkv * 16) return;
    const int c8 = idx & 15, th = idx >> 4;
    const int hk = th % hkv, tok = th / hkv;
    const int key = pos + tok, b = key / BK, kk = key % BK;
    uint8_t* base = kv + ((size_t)hk * nbc + b) * BLOCK_BYTES;
    const size_t src = ((size_t)tok * hkv + hk) * HD + c8 * 8;
    // K: dims 8*c8 .. 8*c8+7 are one 16-byte lane slot of tile (kk/16)*4 + c8/4
    const int c = c8 >> 2, g = c8 & 3;
    *reinterpret_cast<uint4*>(base + ((kk >> 4) * 4 + c) * 1024 + ((kk & 15) + 16 * g) * 16) =
        *reinterpret_cast<const uint4*>(kn + src);
    // V: entry kk sits in lane group gv, element ev of every dimension's slot
    const int half = kk >> 4, w = kk & 15;
    const int gv = w >> 2, ev = (w & 3) + 4 * half;
    const uint4 vv = *reinterpret_cast<const uint4*>(vn + src);
    const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = c8 * 8 + e;
        const uint16_t val = (uint16_t)(vw[e >> 1] >> (16 * (e & 1)));
        *reinterpret_cast<uint16_t*>(base + 8192 + (d >> 4) * 1024 + ((d & 15) + 16 * gv) * 16 + 2 * ev) = val;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int g_bps_override = 0;

struct Plan {
    int nqt, nblk, bps, nsplit;
};

Plan make_plan(int m, int hq, int hkv, int len, int cus) {
    Plan p;
    p.nqt = (m * (hq / hkv) + 15) / 16;
    p.nblk = (len + BK - 1) / BK;
    int bps;
    if (g_bps_override > 0) {
        bps = g_bps_override;
    } else {
        // About one workgroup per two compute units over all heads: a workgroup
        // streams at most ~60 GB/s, so half the units already reach the HBM
        // rate, and fewer ranges keep the merge short.  Ranges hold at least 8
        // blocks (two per wave), and with two query tiles, which merge in two
        // rounds, at least 16 from 128 blocks on (measured with Hq 32, Hkv 8 on
        // 256 units: L = 4096, M = 8 took 16.3 us against 19.1 us with 8-block
        // ranges, on the same part in alternating runs).
        const int cu = cus > 0 ? cus : 256;
        const int per_head = max(1, (cu / 2 + hkv - 1) / hkv);
        bps = (p.nblk + per_head - 1) / per_head;
        const int minb = (p.nqt >= 2 && p.nblk >= 32 * AW) ? 4 * AW : 2 * AW;
        if (bps < minb) bps = minb;
    }
    if (bps > p.nblk) bps = p.nblk;
    if ((p.nblk + bps - 1) / bps > kMaxSplits) bps = (p.nblk + kMaxSplits - 1) / kMaxSplits;
    p.bps = bps;
    p.nsplit = (p.nblk + bps - 1) / bps;
    return p;
}

struct DevState {
    int cus = 0;
    bool lds_set[5] = {false, false, false, false, false};
};
std::mutex g_mu;
DevState g_dev[64];

// Caller-owned workspace: [hdr: 256 B][cnt: kMaxKvHeads u32][flag: kMaxKvHeads *
// kMaxSplits u32] (fixed size, so one buffer serves calls of any shape), then
// the partial states.  Only launches that split the prefix touch it.
constexpr size_t kCountersBytes = ((size_t)kMaxKvHeads * (1 + kMaxSplits) * 4 + 255) / 256 * 256;
constexpr size_t kHeaderBytes = 256 + kCountersBytes;
constexpr int kChunk = PSTRIDE * 16;      // floats of one partial state per query tile

size_t workspace_bytes(const Plan& p, int hkv) {
    return p.nsplit > 1 ? kHeaderBytes + (size_t)hkv * p.nsplit * p.nqt * kChunk * 4 : 0;
}

hipError_t device_cus(int dev, int& cus) {
    std::lock_guard<std::mutex> lk(g_mu);
    DevState& ds = g_dev[dev];
    if (ds.cus == 0) {
        int v = 0;
        hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        ds.cus = v > 0 ? v : 256;
    }
    cus = ds.cus;
    return hipSuccess;
}

// The plan of a call on the current device.
hipError_t current_plan(int m, int hq, int hkv, int len, Plan& p, int& dev) {
    dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int cus = 0;
    e = device_cus(dev, cus);
    if (e != hipSuccess) return e;
    p = make_plan(m, hq, hkv, len, cus);
    return hipSuccess;
}

hipError_t launch_attention(const Plan& p, int dev, const uint16_t* q, int m, int hq, int hkv,
                            const void* kv, int cap, int len, float scale, float* out, void* ws,
                            hipStream_t st) {
    DevState& ds = g_dev[dev];
    hipError_t e = hipSuccess;
    uint8_t* const wsb = static_cast<uint8_t*>(ws);
    AttnArgs a;
    a.q = q;
    a.kv = static_cast<const uint8_t*>(kv);
    a.out = out;
    a.hdr = reinterpret_cast<uint32_t*>(wsb);
    a.cnt = wsb ? reinterpret_cast<uint32_t*>(wsb + 256) : nullptr;
    a.flag = wsb ? a.cnt + kMaxKvHeads : nullptr;
    a.part = wsb ? reinterpret_cast<float*>(wsb + kHeaderBytes) : nullptr;
    a.m = m;
    a.hq = hq;
    a.g = hq / hkv;
    a.r = m * a.g;
    a.len = len;
    a.nbc = cap / BK;
    a.nblk = p.nblk;
    a.bps = p.bps;
    a.nsplit = p.nsplit;
    a.part_bytes = (int)(workspace_bytes(p, hkv) > 0 ? workspace_bytes(p, hkv) - kHeaderBytes : 0);
    a.nwg = p.nsplit * hkv;
    a.sl2 = scale * 1.4426950408889634f;
    void (*fn)(AttnArgs) = nullptr;
    switch (p.nqt) {
        case 1: fn = attn_kernel<1>; break;
        case 2: fn = attn_kernel<2>; break;
        case 3: fn = attn_kernel<3>; break;
        case 4: fn = attn_kernel<4>; break;
        default: return hipErrorInvalidValue;
    }
    const size_t lds = (size_t)AW * p.nqt * 34 * 64 * 4;
    if (lds > 64 * 1024) {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!ds.lds_set[p.nqt]) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            ds.lds_set[p.nqt] = true;
        }
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)p.nsplit, (unsigned)hkv), dim3(AT), lds, st, a);
    return hipGetLastError();
}

// Host copy of the cache layout (the append kernel's mapping, entry by entry).
void pack_host(const uint16_t* k, const uint16_t* v, int hkv, int len, int cap, uint8_t* out) {
    const int nbc = cap / BK;
    std::memset(out, 0, (size_t)hkv * nbc * BLOCK_BYTES);
    for (int hk = 0; hk < hkv; ++hk)
        for (int key = 0; key < len; ++key) {
            const int b = key / BK, kk = key % BK;
            uint8_t* base = out + ((size_t)hk * nbc + b) * BLOCK_BYTES;
            const uint16_t* kr = k + ((size_t)hk * len + key) * HD;
            const uint16_t* vr = v + ((size_t)hk * len + key) * HD;
            const int half = kk >> 4, w = kk & 15;
            const int gv = w >> 2, ev = (w & 3) + 4 * half;
            for (int d = 0; d < HD; ++d) {
                const int c = d / 32, g = (d % 32) / 8, e = d % 8;
                std::memcpy(base + ((half * 4 + c) * 1024 + (w + 16 * g) * 16 + 2 * e), kr + d, 2);
                std::memcpy(base + 8192 + (d >> 4) * 1024 + ((d & 15) + 16 * gv) * 16 + 2 * ev, vr + d, 2);
            }
        }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace ska

SK_EXPORT sk_status sk_kv_append(void* kv, int hkv, int cap, int pos, int t, const uint16_t* k_new,
                                 const uint16_t* v_new, void* stream) {
    if (!kv || !k_new || !v_new) return SK_ERR_NULL;
    if (hkv < 1 || t < 1 || pos < 0 || cap < ska::BK || cap % ska::BK != 0 || (int64_t)pos + t > cap)
        return SK_ERR_SHAPE;
    if (!ska::aligned16(kv) || !ska::aligned16(k_new) || !ska::aligned16(v_new)) return SK_ERR_ALIGN;
    const int64_t n = (int64_t)t * hkv * 16;
    if (n > (int64_t)1 << 30) return SK_ERR_SHAPE;
    hipLaunchKernelGGL(ska::kv_append_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint8_t*>(kv), hkv, cap / ska::BK, pos, t,
                       k_new, v_new);
    return hipGetLastError() == hipSuccess ? SK_OK : SK_ERR_HIP;
}

SK_EXPORT sk_status sk_attention_workspace_size(int m, int hq, int hkv, int len, size_t* bytes) {
    if (!bytes) return SK_ERR_NULL;
    if (m < 1 || m > 8 || hkv < 1 || hq < 1 || hq % hkv != 0 || len < m) return SK_ERR_SHAPE;
    if ((int64_t)m * (hq / hkv) > ska::kMaxRows || hkv > ska::kMaxKvHeads) return SK_ERR_UNSUPPORTED;
    ska::Plan p;
    int dev = 0;
    if (ska::current_plan(m, hq, hkv, len, p, dev) != hipSuccess) return SK_ERR_HIP;
    *bytes = ska::workspace_bytes(p, hkv);
    return SK_OK;
}

SK_EXPORT sk_status sk_decode_attention(const uint16_t* q, int m, int hq, int hkv, const void* kv, int cap,
                                        int len, float scale, float* out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    if (!q || !kv || !out) return SK_ERR_NULL;
    if (m < 1 || m > 8 || hkv < 1 || hq < 1 || hq % hkv != 0 || cap < ska::BK || cap % ska::BK != 0 ||
        len < m || len > cap || !std::isfinite(scale) || !(scale > 0.0f))
        return SK_ERR_SHAPE;
    // rows per KV head; 32-bit offsets into the workspace and into one range
    if ((int64_t)m * (hq / hkv) > ska::kMaxRows || hkv > ska::kMaxKvHeads || cap > ska::kMaxEntries)
        return SK_ERR_UNSUPPORTED;
    if (!ska::aligned16(q) || !ska::aligned16(kv) || !ska::aligned16(out)) return SK_ERR_ALIGN;
    ska::Plan p;
    int dev = 0;
    if (ska::current_plan(m, hq, hkv, len, p, dev) != hipSuccess) return SK_ERR_HIP;
    const size_t need = ska::workspace_bytes(p, hkv);
    if (need > 0 && (!workspace || workspace_bytes < need ||
                     (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0))
        return SK_ERR_WORKSPACE;
    if (need > ((size_t)1 << 31)) return SK_ERR_UNSUPPORTED;     // 32-bit offsets into the partials
    const hipError_t e = ska::launch_attention(p, dev, q, m, hq, hkv, kv, cap, len, scale, out,
                                               need > 0 ? workspace : nullptr,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SK_OK : SK_ERR_HIP;
}

SK_EXPORT sk_status sk_kv_pack_host(const uint16_t* k, const uint16_t* v, int hkv, int len, int cap,
                                    void* out) {
    if (!k || !v || !out) return SK_ERR_NULL;
    if (hkv < 1 || len < 0 || cap < ska::BK || cap % ska::BK != 0 || len > cap) return SK_ERR_SHAPE;
    ska::pack_host(k, v, hkv, len, cap, static_cast<uint8_t*>(out));
    return SK_OK;
}

SK_EXPORT sk_status sk_test_attention_plan(int m, int hq, int hkv, int len, int cus, int* splits,
                                           int* blocks_per_split) {
    if (!splits || !blocks_per_split) return SK_ERR_NULL;
    if (m < 1 || m > 8 || hkv < 1 || hq < 1 || hq % hkv != 0 || len < m) return SK_ERR_SHAPE;
    if (cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || ska::device_cus(dev, cus) != hipSuccess) return SK_ERR_HIP;
    }
    const ska::Plan p = ska::make_plan(m, hq, hkv, len, cus);
    *splits = p.nsplit;
    *blocks_per_split = p.bps;
    return SK_OK;
}

SK_EXPORT sk_status sk_test_set_attention_split(int blocks_per_split) {
    if (blocks_per_split < 0) return SK_ERR_SHAPE;
    ska::g_bps_override = blocks_per_split;
    return SK_OK;
}
