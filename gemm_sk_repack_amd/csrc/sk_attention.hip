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
// The four waves' states are combined through LDS in wave order; with one
// range the workgroup writes O, otherwise it writes its partial state, and
// the last of the KV head's workgroups to arrive (one arrival counter per
// head, release/acquire fences around it) combines the ranges in range order
// and writes O.  Results do not depend on timing.
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
constexpr int kMaxSplits = 128;
constexpr int PSTRIDE = HD + 2;               // floats per partial query row: O[128], max, sum

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct AttnArgs {
    const uint16_t* q;   // [M][Hq][128]
    const uint8_t* kv;   // cache, layout in sk_attention.h
    float* out;          // [M][Hq][128]
    float* part;         // [Hkv][nsplit]{ O [RP][128], (max, sum) [RP][2] }
    uint32_t* cnt;       // [Hkv]
    int m, hq, g, r, len, nbc, nblk, bps, nsplit;
    float sl2;           // scale * log2(e)
};

__device__ inline uint32_t bf16_rne(float f) {
    // f is finite and >= 0 here (a softmax weight or its remainder)
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int NQT>
__global__ __launch_bounds__(AT) void attn_kernel(AttnArgs a) {
    constexpr int RP = NQT * 16;              // query rows padded to whole tiles
    // wave-state exchange: [t][dt*4+v][lane] output values, [t][lane] max and sum;
    // reused by the final merge for the ranges' weights
    __shared__ float xo[NQT * 32 * 64];
    __shared__ float xm[NQT * 64], xl[NQT * 64];
    __shared__ float den[RP];
    __shared__ int last;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int s = blockIdx.x, hk = blockIdx.y;
    const int M = a.m, G = a.g, R = a.r, L = a.len;

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

    // 2. this wave's blocks: b0 + wv, b0 + wv + 4, ... below b1.  Loads go
    //    through a buffer resource covering exactly this range, so the
    //    pipeline's look-ahead loads past the range return zeros without
    //    touching memory and every wave issues the same, static load pattern.
    const int wu = __builtin_amdgcn_readfirstlane(wv);
    const int b0 = s * a.bps;
    const int b1 = min(b0 + a.bps, a.nblk);
    const int nw = (b1 - b0 > wu) ? (b1 - b0 - wu + AW - 1) / AW : 0;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.kv + ((size_t)hk * a.nbc + b0) * BLOCK_BYTES), (short)0,
        (b1 - b0) * BLOCK_BYTES, 0x00020000);

    float mrun[NQT], lrun[NQT];
    v4f o[NQT][8];
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        mrun[t] = -INFINITY;
        lrun[t] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    auto load = [&](uint4 (&kb)[8], uint4 (&vb)[8], int i) {
        const int off = (wu + AW * i) * BLOCK_BYTES + lane * 16;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            kb[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + j * 1024, 0, 0));
#pragma unroll
        for (int j = 0; j < 8; ++j)
            vb[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + 8192 + j * 1024, 0, 0));
    };

    auto compute = [&](const uint4 (&kb)[8], const uint4 (&vin)[8], int i) {
        const int blk = b0 + wu + AW * i;
        const int key0 = blk * BK + 4 * g4;
        uint4 vb[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) vb[dt] = vin[dt];
        if (blk * BK + BK > L) {
            // the prefix ends inside this block: entries at or past L may hold
            // anything (0 * Inf would be NaN), so their V values become zero
            const int nv = L - blk * BK;      // valid entries, 1..31
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
        }
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
                x[v] = (key0 + v <= lim[t]) ? s0[v] * a.sl2 : -INFINITY;
                x[4 + v] = (key0 + 16 + v <= lim[t]) ? s1[v] * a.sl2 : -INFINITY;
            }
            float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                             fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(mrun[t], mx);
            const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(mrun[t] - mu);
            mrun[t] = mnew;
            uint32_t hb[8], lb[8];
            float ps = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = __builtin_amdgcn_exp2f(x[j] - mu);
                ps += p;
                hb[j] = bf16_rne(p);
                lb[j] = bf16_rne(p - __uint_as_float(hb[j] << 16));
            }
            lrun[t] = lrun[t] * alpha + ps;
            const uint4 ph = make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16),
                                        hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16));
            const uint4 pl = make_uint4(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16),
                                        lb[4] | (lb[5] << 16), lb[6] | (lb[7] << 16));
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                o[t][dt] *= alpha;
                o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vb[dt]), as_bf16x8(ph), o[t][dt], 0, 0, 0);
                o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vb[dt]), as_bf16x8(pl), o[t][dt], 0, 0, 0);
            }
        }
    };

    // 3. the wave's blocks, two register slots: the next block's loads are in
    //    flight while a block is computed
    if (nw > 0) {
        uint4 k0[8], v0[8], k1[8], v1[8];
        load(k0, v0, 0);
        load(k1, v1, 1);
        for (int i = 0; i < nw; i += 2) {
            compute(k0, v0, i);
            load(k0, v0, i + 2);
            if (i + 1 < nw) compute(k1, v1, i + 1);
            load(k1, v1, i + 3);
        }
    }
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
        lrun[t] += __shfl_xor(lrun[t], 16);
        lrun[t] += __shfl_xor(lrun[t], 32);
    }

    // 4. combine the waves' states in wave order (wave 0 accumulates)
    for (int src = 1; src < AW; ++src) {
        if (wv == src) {
#pragma unroll
            for (int t = 0; t < NQT; ++t) {
                xm[t * 64 + lane] = mrun[t];
                xl[t * 64 + lane] = lrun[t];
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) xo[(t * 32 + dt * 4 + v) * 64 + lane] = o[t][dt][v];
            }
        }
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int t = 0; t < NQT; ++t) {
                const float mb = xm[t * 64 + lane], lb = xl[t * 64 + lane];
                const float mn = fmaxf(mrun[t], mb);
                const float mu = (mn == -INFINITY) ? 0.0f : mn;
                const float wa = __builtin_amdgcn_exp2f(mrun[t] - mu);
                const float wb = __builtin_amdgcn_exp2f(mb - mu);
                mrun[t] = mn;
                lrun[t] = __builtin_fmaf(lb, wb, lrun[t] * wa);
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        o[t][dt][v] = __builtin_fmaf(xo[(t * 32 + dt * 4 + v) * 64 + lane], wb, o[t][dt][v] * wa);
            }
        }
        __syncthreads();
    }

    // 5. one range: write O.  Otherwise store the partial state; the last
    //    workgroup of this head to arrive merges.
    if (a.nsplit == 1) {
        if (wv == 0) {
#pragma unroll
            for (int t = 0; t < NQT; ++t) {
                const int r = t * 16 + l16;
                if (r < R) {
                    const int mm = r / G, hg = r - mm * G;
                    const float inv = 1.0f / lrun[t];
                    float* op = a.out + (size_t)(mm * a.hq + hk * G + hg) * HD + 4 * g4;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt)
                        *reinterpret_cast<float4*>(op + dt * 16) =
                            make_float4(o[t][dt][0] * inv, o[t][dt][1] * inv, o[t][dt][2] * inv, o[t][dt][3] * inv);
                }
            }
        }
        return;
    }

    // this head's partials: per range, O [RP][128] then (max, sum) [RP][2]
    constexpr int CH = RP * PSTRIDE;
    float* const hpart = a.part + (size_t)hk * a.nsplit * CH;
    if (wv == 0) {
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
            const int r = t * 16 + l16;
            if (r < R) {
                float* pp = hpart + (size_t)s * CH + r * HD + 4 * g4;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    *reinterpret_cast<float4*>(pp + dt * 16) = make_float4(o[t][dt][0], o[t][dt][1], o[t][dt][2], o[t][dt][3]);
                if (g4 == 0)
                    *reinterpret_cast<float2*>(hpart + (size_t)s * CH + RP * HD + 2 * r) = make_float2(mrun[t], lrun[t]);
            }
        }
        __threadfence();                      // release: the partial before the arrival
        if (lane == 0) {
            const uint32_t old = __hip_atomic_fetch_add(&a.cnt[hk], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int lst = old == (uint32_t)(a.nsplit - 1);
            if (lst) __hip_atomic_store(&a.cnt[hk], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = lst;
        }
    }
    __syncthreads();
    if (!last) return;
    __threadfence();                          // acquire: every range's partial is visible

    // 6. merge the ranges in range order: weights exp2(max_s - max) per (range, row)
    float* const wts = xo;                    // [nsplit][RP]
    if (tid < R) {
        float mx = -INFINITY;
        for (int q = 0; q < a.nsplit; ++q) mx = fmaxf(mx, hpart[(size_t)q * CH + RP * HD + 2 * tid]);
        float d = 0.0f;
        for (int q = 0; q < a.nsplit; ++q) {
            const float2 ml = *reinterpret_cast<const float2*>(hpart + (size_t)q * CH + RP * HD + 2 * tid);
            const float w = __builtin_amdgcn_exp2f(ml.x - mx);
            wts[q * RP + tid] = w;
            d = __builtin_fmaf(ml.y, w, d);
        }
        den[tid] = 1.0f / d;
    }
    __syncthreads();
    for (int it = tid; it < R * (HD / 4); it += AT) {
        const int r = it / (HD / 4), d4 = it - r * (HD / 4);
        const float* pp = hpart + (size_t)r * HD + 4 * d4;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        auto add = [&](const float4 v, const float w) {
            acc.x = __builtin_fmaf(v.x, w, acc.x);
            acc.y = __builtin_fmaf(v.y, w, acc.y);
            acc.z = __builtin_fmaf(v.z, w, acc.z);
            acc.w = __builtin_fmaf(v.w, w, acc.w);
        };
        int q = 0;
        for (; q + 4 <= a.nsplit; q += 4) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(pp + (size_t)(q + u) * CH);
#pragma unroll
            for (int u = 0; u < 4; ++u) add(v[u], wts[(q + u) * RP + r]);
        }
        for (; q < a.nsplit; ++q) add(*reinterpret_cast<const float4*>(pp + (size_t)q * CH), wts[q * RP + r]);
        const int mm = r / G, hg = r - mm * G;
        const float dn = den[r];
        *reinterpret_cast<float4*>(a.out + (size_t)(mm * a.hq + hk * G + hg) * HD + 4 * d4) =
            make_float4(acc.x * dn, acc.y * dn, acc.z * dn, acc.w * dn);
    }
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
        // about two workgroups per compute unit over all heads, at least one
        // block per wave
        const int target = 2 * (cus > 0 ? cus : 256);
        const int per_head = (target + hkv - 1) / hkv;
        bps = (p.nblk + per_head - 1) / per_head;
        if (bps < AW) bps = AW;
    }
    if (bps > p.nblk) bps = p.nblk;
    if ((p.nblk + bps - 1) / bps > kMaxSplits) bps = (p.nblk + kMaxSplits - 1) / kMaxSplits;
    p.bps = bps;
    p.nsplit = (p.nblk + bps - 1) / bps;
    return p;
}

struct DevState {
    int cus = 0;
    void* ws = nullptr;        // [cnt: cap_h uint32, padded to 256 B][part: cap_part floats]
    int cap_h = 0;
    size_t cap_part = 0;
};
std::mutex g_mu;
DevState g_dev[64];

hipError_t device_cus(int dev, int& cus) {
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

hipError_t launch_attention(const uint16_t* q, int m, int hq, int hkv, const void* kv, int cap, int len,
                            float scale, float* out, hipStream_t st) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int cus = 0;
    e = device_cus(dev, cus);
    if (e != hipSuccess) return e;
    const Plan p = make_plan(m, hq, hkv, len, cus);
    const size_t part_floats = p.nsplit > 1 ? (size_t)hkv * p.nsplit * p.nqt * 16 * PSTRIDE : 0;
    DevState& ds = g_dev[dev];
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!ds.ws || ds.cap_h < hkv || ds.cap_part < part_floats) {
            const int cap_h = ds.cap_h > hkv ? ds.cap_h : (hkv > 64 ? hkv : 64);
            const size_t cap_part = ds.cap_part > part_floats ? ds.cap_part : part_floats;
            if (ds.ws) {
                e = hipDeviceSynchronize();
                if (e != hipSuccess) return e;
                (void)hipFree(ds.ws);
                ds.ws = nullptr;
            }
            const size_t cnt_bytes = ((size_t)cap_h * 4 + 255) / 256 * 256;
            const size_t bytes = cnt_bytes + cap_part * 4;
            e = hipMalloc(&ds.ws, bytes);
            if (e != hipSuccess) return e;
            e = hipMemset(ds.ws, 0, bytes);
            if (e != hipSuccess) return e;
            e = hipDeviceSynchronize();
            if (e != hipSuccess) return e;
            ds.cap_h = cap_h;
            ds.cap_part = cap_part;
        }
    }
    AttnArgs a;
    a.q = q;
    a.kv = static_cast<const uint8_t*>(kv);
    a.out = out;
    a.cnt = static_cast<uint32_t*>(ds.ws);
    a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ds.ws) + ((size_t)ds.cap_h * 4 + 255) / 256 * 256);
    a.m = m;
    a.hq = hq;
    a.g = hq / hkv;
    a.r = m * a.g;
    a.len = len;
    a.nbc = cap / BK;
    a.nblk = p.nblk;
    a.bps = p.bps;
    a.nsplit = p.nsplit;
    a.sl2 = scale * 1.4426950408889634f;
    void (*fn)(AttnArgs) = nullptr;
    switch (p.nqt) {
        case 1: fn = attn_kernel<1>; break;
        case 2: fn = attn_kernel<2>; break;
        case 3: fn = attn_kernel<3>; break;
        case 4: fn = attn_kernel<4>; break;
        default: return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)p.nsplit, (unsigned)hkv), dim3(AT), 0, st, a);
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

SK_EXPORT sk_status sk_decode_attention(const uint16_t* q, int m, int hq, int hkv, const void* kv, int cap,
                                        int len, float scale, float* out, void* stream) {
    if (!q || !kv || !out) return SK_ERR_NULL;
    if (m < 1 || m > 8 || hkv < 1 || hq < 1 || hq % hkv != 0 || cap < ska::BK || cap % ska::BK != 0 ||
        len < m || len > cap || !std::isfinite(scale) || !(scale > 0.0f))
        return SK_ERR_SHAPE;
    if ((int64_t)m * (hq / hkv) > ska::kMaxRows || hkv > 65535) return SK_ERR_UNSUPPORTED;
    if (!ska::aligned16(q) || !ska::aligned16(kv) || !ska::aligned16(out)) return SK_ERR_ALIGN;
    const hipError_t e = ska::launch_attention(q, m, hq, hkv, kv, cap, len, scale, out,
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
