// sk_gemm.hip -- skinny quantized GEMM kernels for gfx950 (MI355X).
//
//   y[m][n] = sx[m] * sum_j s[n][j] * P[m][n][j],   m < M <= 8,
//   P[m][n][j] = sum_{k in group j} w[n][k] * q[m][k]          (exact int32)
//
// ("Doubling the LLM token rate in ComfyUI", section on optimizing linear
// kernels; "Comfy quantization formats", sections on weight formats and on
// activations.)  One launch does everything.  The grid holds one 1024-thread
// workgroup per compute unit; workgroup p works on K-slice s = p / R of the
// weight (S slices) for a contiguous range of 16-row tiles, so it needs the
// activations of its own slice only.
//
//  1. Load this thread's activations (registers), then issue the first PIPE
//     super-blocks of the weight stream.  Every load is unconditional (an
//     out-of-range slot reads a harmless in-bounds address), so the number of
//     outstanding loads is known at compile time and waiting for the
//     activations never waits for the weight stream.
//  2. Activation prologue while the weights are in flight: optional RMSNorm or
//     SwiGLU; per-row statistics.  With S > 1 the full-row sum of squares and
//     absmax are exchanged between slices through tagged device-scope words
//     (one wave publishes and polls before it issues its own weight loads;
//     the wait is bounded and a time-out falls back to computing the missing
//     slices locally).  Then sx = absmax/127 and q = rint(h/sx) -> int8 in LDS,
//     plus the per-group sums of q that undo the offset-binary weight codes.
//  3. Stream the tiles through a register pipeline.  M >= 2 uses
//     v_mfma_i32_16x16x32_i8 (q = A operand, M padded to 16; weights = B);
//     M = 1 uses v_dot4_i32_i8.  The offset correction is the accumulator's
//     initial value, so the integer result is the exact per-group partial; it
//     is scaled by the FP32 group scale and accumulated in fp32.
//  4. Per tile, the waves' sums are added in a fixed order through LDS.  With
//     S = 1 the workgroup writes y.  Otherwise it stores a tagged partial; at
//     the end, the last of a tile's S workgroups to arrive adds the S
//     partials in slice order and writes y.  No floating-point atomics and no
//     cache-flushing fences: results are deterministic.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sk_internal.h"

namespace sk {

namespace {

constexpr int NW = 16;         // waves per workgroup
constexpr int NT = NW * 64;    // threads per workgroup
constexpr int PIPE = 4;        // super-blocks in flight per wave
constexpr int PRIME = 2;       // of which issued before the activation prologue
constexpr int MO = 2;          // activation octets per thread
constexpr int SMAX = 32;       // largest number of K-slices
constexpr int kMaxTilesPerGroup = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;
struct KArgs {
    const uint8_t* data;
    const void* x;
    const void* x2;
    int64_t ld;
    const float* gamma;
    float eps;
    float* y;
    int8_t* q_out;
    float* sx_out;
    int32_t* p_out;
    WsHeader* ws;
    uint32_t* cnt;
    u64* part;
    int n, k, m;
    int T, KB, kg;
    int sb_row, wsb_row;
    int64_t tile_full;
    int S, R, P, TW, KW, spw, KBs, KS, WPR, ks;
    int spin_limit;
};

struct Smem {
    double wd[NW];
    float wf[NW];
    double exd[SMAX * 8];
    float exf[SMAX * 8];
    float sx[8];
    float inv[8];
    float rr[8];
    int miss[SMAX];
    uint32_t tag;
    int last[kMaxTilesPerGroup];
};

// --------------------------------------------------------------------------
// activation helpers
// --------------------------------------------------------------------------

template <int XT>
__device__ inline void load8(const void* base, int64_t off, float v[8]) {
    if (XT == 0) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
}

#pragma clang fp contract(off)

// e^x as one fixed fp32 operation sequence: Cody-Waite reduction by ln 2 split
// into a short high part and a low part, degree-7 Taylor polynomial of e^r on
// |r| <= ln2/2 in Horner form, then scaling by 2^n in two exact-then-rounded
// steps.  Each operation is rounded separately (no contraction).
__device__ inline float sk_expf(float x) {
    if (x >= 89.0f) return __builtin_inff();
    if (x <= -104.0f) return 0.0f;
    const float kLog2e = (float)1.4426950408889634;
    const float kLn2Hi = 0.693359375f;
    const float kLn2Lo = (float)(0.6931471805599453 - 0.693359375);
    float n = __builtin_rintf(x * kLog2e);
    float r = (x - n * kLn2Hi) - n * kLn2Lo;
    float p = (float)(1.0 / 5040.0);
    p = p * r + (float)(1.0 / 720.0);
    p = p * r + (float)(1.0 / 120.0);
    p = p * r + (float)(1.0 / 24.0);
    p = p * r + (float)(1.0 / 6.0);
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    int ni = (int)n;
    int e1 = ni >> 1;          // floor(n / 2)
    int e2 = ni - e1;
    return (p * __int_as_float((e1 + 127) << 23)) * __int_as_float((e2 + 127) << 23);
}

__device__ inline float silu_mul(float g, float u) {
    float den = 1.0f + sk_expf(-g);
    float s = g / den;
    return s * u;
}

__device__ inline float rms_apply(float x, float r, float g) {
    float t = x * r;
    return t * g;
}

// q = clamp(rint(fp32(h / sx)), -127, 127), bit-exactly, for sx > 0.
// t = h * inv with inv = fp32(1/sx) is within |h/sx| * 2^-23 (< 1.6e-5 here)
// of h/sx, and fp32(h/sx) within half an ulp (<= 2^-18) of it, so rint(t)
// equals rint(fp32(h/sx)) unless t lies within 2e-5 of a half-integer; only
// then (or for a tiny sx) is the quotient formed by IEEE division.
__device__ inline int quant1(float h, float sx, float inv, bool exact_row) {
    float t = h * inv;
    float r = __builtin_rintf(t);
    if (exact_row || fabsf(t - r) > 0.49998f) {
        t = h / sx;
        r = __builtin_rintf(t);
    }
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

#pragma clang fp contract(on)

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Thread -> activation mapping: row m = wave / WPR (WPR waves per row); the
// thread's octets of the slice are it and it + TPR (it = index in the row).
struct ActMap {
    int m;       // row, or >= M if the thread holds no activations
    int it;      // index within the row's threads
    int tpr;     // threads per row
};

__device__ inline ActMap act_map(const KArgs& a, int wv, int lane) {
    ActMap am;
    am.m = wv / a.WPR;
    am.it = (wv % a.WPR) * 64 + lane;
    am.tpr = a.WPR * 64;
    return am;
}

__device__ inline bool oct_valid(const KArgs& a, const ActMap& am, int i) {
    return am.m < a.m && am.it + i * am.tpr < (a.KS >> 3);
}

// Raw activations of slice [k_lo, k_lo + KS) (SwiGLU: gate in xv, up in uv).
// Unconditional loads: an invalid octet reads element 0 and is zeroed later.
template <int PRO, int XT>
__device__ inline void load_act(const KArgs& a, const ActMap& am, int k_lo, float xv[MO][8],
                                float uv[MO][8]) {
#pragma unroll
    for (int i = 0; i < MO; ++i) {
        const bool ok = oct_valid(a, am, i);
        const int64_t off = ok ? (int64_t)am.m * a.ld + k_lo + 8 * (am.it + i * am.tpr) : 0;
        load8<XT>(a.x, off, xv[i]);
        if (PRO == PRO_SWIGLU) load8<XT>(a.x2, off, uv[i]);
    }
}

// Turn loaded raw values into h (SwiGLU) and zero invalid octets.
template <int PRO>
__device__ inline void finish_act(const KArgs& a, const ActMap& am, float xv[MO][8], float uv[MO][8]) {
#pragma unroll
    for (int i = 0; i < MO; ++i) {
        const bool ok = oct_valid(a, am, i);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float h = xv[i][e];
            if (PRO == PRO_SWIGLU) h = silu_mul(xv[i][e], uv[i][e]);
            xv[i][e] = ok ? h : 0.0f;
        }
    }
}

__device__ inline void row_sum_d(Smem& sm, int wv, int lane, double v) {
    v = wave_sum(v);
    if (lane == 0) sm.wd[wv] = v;
}
__device__ inline void row_max_f(Smem& sm, int wv, int lane, float v) {
    v = wave_max(v);
    if (lane == 0) sm.wf[wv] = v;
}
__device__ inline double combine_d(const KArgs& a, const Smem& sm, int m) {
    double s = 0.0;
    for (int w = m * a.WPR; w < (m + 1) * a.WPR; ++w) s += sm.wd[w];
    return s;
}
__device__ inline float combine_f(const KArgs& a, const Smem& sm, int m) {
    float s = 0.0f;
    for (int w = m * a.WPR; w < (m + 1) * a.WPR; ++w) s = fmaxf(s, sm.wf[w]);
    return s;
}

// Statistics of slice `sl`, computed locally when its exchange word did not
// arrive in time.  Same thread mapping and summation order as the workgroups
// that own that slice, so the result is bit-identical.  All threads call it.
template <int PRO, int XT>
__device__ inline void slice_stat(const KArgs& a, Smem& sm, int wv, int lane, int sl, bool want_ss) {
    const ActMap am = act_map(a, wv, lane);
    float xv[MO][8], uv[MO][8];
    load_act<PRO, XT>(a, am, sl * a.KS, xv, uv);
    finish_act<PRO>(a, am, xv, uv);
    if (want_ss) {
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < MO; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += (double)xv[i][e] * (double)xv[i][e];
        row_sum_d(sm, wv, lane, ss);
    } else {
        float mx = 0.0f;
        const float r = (am.m < a.m) ? sm.rr[am.m] : 1.0f;
#pragma unroll
        for (int i = 0; i < MO; ++i) {
            const int k0 = sl * a.KS + 8 * (am.it + i * am.tpr);
            const bool ok = oct_valid(a, am, i);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float h = xv[i][e];
                if (PRO == PRO_RMSNORM && ok) h = rms_apply(h, r, a.gamma[k0 + e]);
                mx = fmaxf(mx, fabsf(h));
            }
        }
        row_max_f(sm, wv, lane, mx);
    }
    __syncthreads();
    if (threadIdx.x < a.m) {
        if (want_ss) sm.exd[sl * 8 + threadIdx.x] = combine_d(a, sm, threadIdx.x);
        else sm.exf[sl * 8 + threadIdx.x] = combine_f(a, sm, threadIdx.x);
    }
    __syncthreads();
}

// Exchange this slice's per-row value with the other slices (S > 1), run by
// the poller wave only.  Every word carries the call's tag in its high half,
// so no fence is needed: a reader simply waits until all words show the tag.
// absmax: one word (tag | float bits).  Sum of squares (double): two words
// (tag | high half), (tag | low half).
__device__ inline void exchange_poll(const KArgs& a, Smem& sm, int lane, int s, bool is_ss) {
    const uint32_t tag = sm.tag;
    if (lane < a.m) {
        const int slot = s * 8 + lane;
        if (is_ss) {
            const u64 bits = (u64)__double_as_longlong(sm.exd[slot]);
            __hip_atomic_store(&a.ws->ssh[slot], ((u64)tag << 32) | (bits >> 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.ws->ssl[slot], ((u64)tag << 32) | (bits & 0xFFFFFFFFull),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            __hip_atomic_store(&a.ws->amax[slot], ((u64)tag << 32) | __float_as_uint(sm.exf[slot]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (lane < SMAX) sm.miss[lane] = 0;
    for (int j = lane; j < a.S * a.m; j += 64) {
        const int sl = j / a.m, mm = j % a.m;
        const int slot = sl * 8 + mm;
        if (sl == s) continue;
        bool ok = false;
        for (int it = 0; it < a.spin_limit; ++it) {
            if (is_ss) {
                const u64 hi = __hip_atomic_load(&a.ws->ssh[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const u64 lo = __hip_atomic_load(&a.ws->ssl[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((uint32_t)(hi >> 32) == tag && (uint32_t)(lo >> 32) == tag) {
                    sm.exd[slot] = __longlong_as_double((long long)(((hi & 0xFFFFFFFFull) << 32) |
                                                                    (lo & 0xFFFFFFFFull)));
                    ok = true;
                    break;
                }
            } else {
                const u64 v = __hip_atomic_load(&a.ws->amax[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((uint32_t)(v >> 32) == tag) {
                    sm.exf[slot] = __uint_as_float((uint32_t)v);
                    ok = true;
                    break;
                }
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (!ok) sm.miss[sl] = 1;          // every writer stores the same value
    }
}

// --------------------------------------------------------------------------
// the kernel
// --------------------------------------------------------------------------

template <int FMT, int PRO, int XT, int GS, bool DOT4>
__global__ __launch_bounds__(NT) void gemm_kernel(KArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ Smem sm;
    constexpr int NG = 4 / GS;                  // groups per super-block
    constexpr int OFF = (FMT == FMT_W6) ? 32 : 8;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int nl = lane & 15;
    const int hl = lane >> 4;
    const int M = a.m;

    // work assignment
    const int s = blockIdx.x / a.R;
    const int r = blockIdx.x % a.R;
    const int k_lo = s * a.KS;
    const int kb_lo = s * a.KBs;
    const int64_t t_begin = (int64_t)r * a.T / a.R;
    const int64_t t_end = (int64_t)(r + 1) * a.T / a.R;
    const int ntile = (int)(t_end - t_begin);
    const int tg = wv / a.KW;                   // tile group of this wave (idle if >= TW)
    const int kw = wv % a.KW;
    const int jn = (ntile + a.TW - 1) / a.TW;   // tiles per group (padded)
    const int jall = jn * a.spw;                // iterations every wave runs
    // With S > 1 the last wave only runs the cross-slice exchange: it never has
    // weight loads in flight, so its polls are not queued behind them.
    const bool poller = (a.S > 1) && (wv == NW - 1);
    const bool active = tg < a.TW && !poller;

    // LDS: [q: M x ks int8][sums of q][wave partials]
    const int KS8 = a.KS >> 3;
    int8_t* q_l = reinterpret_cast<int8_t*>(lds);
    int32_t* qs_l = reinterpret_cast<int32_t*>(lds + (size_t)M * a.ks);
    const int qs_n = DOT4 ? KS8 : (a.KS / (32 * GS)) * 8;
    float* red_l = reinterpret_cast<float*>(qs_l + qs_n);                        // 2 x [NW][8][16]

    auto tile_of = [&](int i) -> int64_t { return t_begin + tg + (int64_t)(i / a.spw) * a.TW; };

    // One super-block's loads into registers.  Always exactly the same load
    // instructions; slots outside the work read the weight's first bytes.
    // Branch-free address arithmetic of super-block slot i (selects only, so the
    // loads issue back to back); an invalid slot reads the weight's first bytes.
    auto addr = [&](int i, bool real, int64_t& wp, int64_t& sp, int& nr) -> bool {
        const int64_t t = tile_of(i);
        const bool valid = real && active && i < jall && t < t_end;
        const int kb = kb_lo + kw * a.spw + i % a.spw;
        const int64_t rem = (int64_t)a.n - t * TILE_ROWS;
        nr = rem < TILE_ROWS ? (int)rem : TILE_ROWS;
        const bool full = nr == TILE_ROWS;
        const int64_t tb = t * a.tile_full;
        wp = tb + (int64_t)kb * nr * (full ? a.sb_row : a.wsb_row);
        sp = full ? wp + nr * a.wsb_row
                  : tb + (int64_t)a.KB * nr * a.wsb_row + (int64_t)kb * nr * NG * 4;
        return valid;
    };
    // slot i into registers (the steady-state pipeline)
    auto load = [&](int i, uint4& w4, uint2& h2, float4& sv) {
        int64_t wp, sp;
        int nr;
        const bool ok = addr(i, true, wp, sp, nr) && nl < nr;
        const int64_t woff = ok ? wp + (hl * nr + nl) * 16 : 0;
        const int64_t hoff = ok ? wp + nr * 64 + (hl * nr + nl) * 8 : 0;
        const int64_t soff = ok ? sp + nl * NG * 4 : 0;
        w4 = *reinterpret_cast<const uint4*>(a.data + woff);
        if (FMT == FMT_W6) h2 = *reinterpret_cast<const uint2*>(a.data + hoff);
        if (NG == 4) {
            sv = *reinterpret_cast<const float4*>(a.data + soff);
        } else if (NG == 2) {
            const float2 v = *reinterpret_cast<const float2*>(a.data + soff);
            sv = make_float4(v.x, v.y, 0.0f, 0.0f);
        } else {
            sv = make_float4(*reinterpret_cast<const float*>(a.data + soff), 0.0f, 0.0f, 0.0f);
        }
    };
    // 1. the call's tag, the activations, then the weight stream (in this order:
    //    a wave's loads complete in issue order, so anything waited on before the
    //    weights arrive must be issued before them)
    const uint32_t gen = __hip_atomic_load(&a.ws->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const ActMap am = act_map(a, wv, lane);
    float xv[MO][8], uv[MO][8], gv[MO][8];
    load_act<PRO, XT>(a, am, k_lo, xv, uv);
    if (PRO == PRO_RMSNORM) {
#pragma unroll
        for (int i = 0; i < MO; ++i) {
            const int64_t off = oct_valid(a, am, i) ? k_lo + 8 * (am.it + i * am.tpr) : 0;
            const float4* gp = reinterpret_cast<const float4*>(a.gamma + off);
            const float4 g0 = gp[0], g1 = gp[1];
            gv[i][0] = g0.x; gv[i][1] = g0.y; gv[i][2] = g0.z; gv[i][3] = g0.w;
            gv[i][4] = g1.x; gv[i][5] = g1.y; gv[i][6] = g1.z; gv[i][7] = g1.w;
        }
    }
    // The first PRIME slots.  Every wave issues the same load instructions (the
    // poller and idle waves read dummies), so the compiler's wait counts are exact.
    uint4 wbuf[PIPE];
    uint2 hbuf[PIPE];
    float4 sbuf[PIPE];
#pragma unroll
    for (int d = 0; d < PRIME; ++d) load(d, wbuf[d], hbuf[d], sbuf[d]);

    // 2. activation prologue
    if (tid == 0) sm.tag = gen + 1u;
    for (int i = tid; i < qs_n; i += NT) qs_l[i] = 0;
    finish_act<PRO>(a, am, xv, uv);

    if (PRO == PRO_RMSNORM) {
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < MO; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += (double)xv[i][e] * (double)xv[i][e];
        row_sum_d(sm, wv, lane, ss);
        __syncthreads();
        if (tid < M) sm.exd[s * 8 + tid] = combine_d(a, sm, tid);
        __syncthreads();
        if (a.S > 1) {
            if (poller) exchange_poll(a, sm, lane, s, true);
            __syncthreads();
            for (int sl = 0; sl < a.S; ++sl)
                if (sm.miss[sl]) slice_stat<PRO, XT>(a, sm, wv, lane, sl, true);
        }
        if (tid < M) {
            double tot = 0.0;
            for (int sl = 0; sl < a.S; ++sl) tot += sm.exd[sl * 8 + tid];
            const float ms = (float)(tot / (double)a.k);
            const float d = ms + a.eps;
            const float sd = (float)__builtin_sqrt((double)d);   // correctly rounded fp32 sqrt
            sm.rr[tid] = (float)(1.0 / (double)sd);               // correctly rounded fp32 1/x
        }
        __syncthreads();
        if (am.m < M) {
            const float rm = sm.rr[am.m];
#pragma unroll
            for (int i = 0; i < MO; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) xv[i][e] = rms_apply(xv[i][e], rm, gv[i][e]);
        }
    }
    {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < MO; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(xv[i][e]));
        row_max_f(sm, wv, lane, mx);
        __syncthreads();
        if (tid < M) sm.exf[s * 8 + tid] = combine_f(a, sm, tid);
        __syncthreads();
        if (a.S > 1) {
            if (poller) exchange_poll(a, sm, lane, s, false);
            __syncthreads();
            for (int sl = 0; sl < a.S; ++sl)
                if (sm.miss[sl]) slice_stat<PRO, XT>(a, sm, wv, lane, sl, false);
        }
        if (tid < 8) {
            float amx = 0.0f;
            if (tid < M)
                for (int sl = 0; sl < a.S; ++sl) amx = fmaxf(amx, sm.exf[sl * 8 + tid]);
            const float sx = amx / 127.0f;
            sm.sx[tid] = (amx > 0.0f) ? sx : 0.0f;
            sm.inv[tid] = (amx > 0.0f) ? 1.0f / sx : 0.0f;
            if (a.sx_out && blockIdx.x == 0 && tid < M) a.sx_out[tid] = sm.sx[tid];
        }
        __syncthreads();
    }

    // quantise this slice into LDS
    if (am.m < M) {
        const float sx = sm.sx[am.m];
        const float inv = sm.inv[am.m];
        const bool exact_row = sx < 2.3509887e-38f;       // 2^-125: 1/sx may not be normal
#pragma unroll
        for (int i = 0; i < MO; ++i) {
            const int o = am.it + i * am.tpr;
            if (o < KS8) {
                uint32_t lo = 0, hi = 0;
                int sum = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int qi = (sx > 0.0f) ? quant1(xv[i][e], sx, inv, exact_row) : 0;
                    sum += qi;
                    const uint32_t b = (uint32_t)(qi & 0xFF);
                    if (e < 4) lo |= b << (8 * e); else hi |= b << (8 * (e - 4));
                }
                *reinterpret_cast<uint2*>(q_l + am.m * a.ks + 8 * o) = make_uint2(lo, hi);
                if (a.q_out && r == 0)
                    *reinterpret_cast<uint2*>(a.q_out + (int64_t)am.m * a.k + k_lo + 8 * o) =
                        make_uint2(lo, hi);
                if (DOT4) qs_l[o] = sum;
                else atomicAdd(&qs_l[(8 * o / (32 * GS)) * 8 + am.m], sum);
            }
        }
    }
    __syncthreads();

#pragma unroll
    for (int d = PRIME; d < PIPE; ++d) load(d, wbuf[d], hbuf[d], sbuf[d]);

    // 3. stream the weights: a register pipeline of PIPE slots in flight
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int ml = nl;   // A-operand row (activation row m) of this lane
    const int iters = (jall + PIPE - 1) / PIPE * PIPE;
    // consume super-block slot i (weights w_in/h_in, scales s_in), then the tile
    // epilogue when slot i is the last one of its tile
    auto process = [&](int i, const uint4 w_in, const uint2 h_in, const float4 s_in) {
        const int64_t t = tile_of(i);
        const int slot_i = i % a.spw;
        if (active && i < jall && t < t_end) {
            const int kbr = kw * a.spw + slot_i;          // super-block within the slice
            const int kb = kb_lo + kbr;
            const int64_t rem = (int64_t)a.n - t * TILE_ROWS;
            const int nr = rem < TILE_ROWS ? (int)rem : TILE_ROWS;
            const bool row_ok = nl < nr;
            const uint32_t wd[4] = {row_ok ? w_in.x : 0u, row_ok ? w_in.y : 0u,
                                    row_ok ? w_in.z : 0u, row_ok ? w_in.w : 0u};
            const float s4[4] = {s_in.x, s_in.y, s_in.z, s_in.w};
            float sv[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) sv[g] = row_ok ? s4[g] : 0.0f;
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lo[j] = wd[j] & 0x0F0F0F0Fu;
                hi[j] = (wd[j] >> 4) & 0x0F0F0F0Fu;
                if (FMT == FMT_W6) {
                    const uint32_t hd = row_ok ? ((j < 2) ? h_in.x : h_in.y) : 0u;
                    if ((j & 1) == 0) {
                        lo[j] |= (hd << 4) & 0x30303030u;
                        hi[j] |= (hd << 2) & 0x30303030u;
                    } else {
                        lo[j] |= hd & 0x30303030u;
                        hi[j] |= (hd >> 2) & 0x30303030u;
                    }
                }
            }
            const int kbase = kbr * 128;          // slice-relative k of this super-block
            if (DOT4) {
                int pj[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k0 = kbase + 32 * j + 8 * hl;
                    const uint2 qv = *reinterpret_cast<const uint2*>(q_l + k0);
                    int c = -OFF * qs_l[k0 >> 3];
                    c = __builtin_amdgcn_sdot4((int)hi[j], (int)qv.y, c, false);
                    pj[j] = __builtin_amdgcn_sdot4((int)lo[j], (int)qv.x, c, false);
                }
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    int pg = 0;
#pragma unroll
                    for (int jj = 0; jj < GS; ++jj) pg += pj[gi * GS + jj];
                    acc[0] = __builtin_fmaf(sv[gi], (float)pg, acc[0]);
                    if (a.p_out && row_ok)
                        atomicAdd(&a.p_out[(t * TILE_ROWS + nl) * a.kg + kb * NG + gi], pg);
                }
            } else {
                long av[4], bv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bv[j] = (long)((uint64_t)lo[j] | ((uint64_t)hi[j] << 32));
                    av[j] = (ml < M) ? *reinterpret_cast<const long*>(
                                           q_l + ml * a.ks + kbase + 32 * j + 8 * hl)
                                     : 0L;
                }
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const int ggl = kbr * NG + gi;    // slice-relative group
                    v4i c = {0, 0, 0, 0};
                    if (hl < 2) {
                        const int4 qv = *reinterpret_cast<const int4*>(qs_l + ggl * 8 + 4 * hl);
                        c[0] = -OFF * qv.x; c[1] = -OFF * qv.y;
                        c[2] = -OFF * qv.z; c[3] = -OFF * qv.w;
                    }
#pragma unroll
                    for (int jj = 0; jj < GS; ++jj)
                        c = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[gi * GS + jj],
                                                                 bv[gi * GS + jj], c, 0, 0, 0);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        acc[rr] = __builtin_fmaf(sv[gi], (float)c[rr], acc[rr]);
                        const int mm = 4 * hl + rr;
                        if (a.p_out && mm < M && row_ok)
                            a.p_out[((int64_t)mm * a.n + t * TILE_ROWS + nl) * a.kg +
                                    kb * NG + gi] = c[rr];
                    }
                }
            }
        }
        if (i < jall && slot_i == a.spw - 1) {
            // 4. tile epilogue: fixed-order sum of the waves' partials.  The partials
            //    buffer alternates between two halves, so one barrier per tile is enough
            //    (a wave cannot reuse a half before every thread passed the next barrier).
            const int j = i / a.spw;
            float* red = red_l + (j & 1) * (NW * 128);
            if (DOT4) {
                red[(wv * 4 + hl) * 16 + nl] = acc[0];
            } else {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int mm = 4 * hl + rr;
                    if (mm < M) red[(wv * 8 + mm) * 16 + nl] = acc[rr];
                }
            }
            __syncthreads();
            const int nout = a.TW * M * 16;
            if (tid < nout) {
                const int ogrp = tid / (M * 16);
                const int omm = (tid / 16) % M;
                const int onn = tid & 15;
                const int64_t ot = t_begin + ogrp + (int64_t)j * a.TW;
                if (ot < t_end) {
                    float osum = 0.0f;
                    const int w0 = ogrp * a.KW;
                    if (DOT4) {
                        for (int w = w0; w < w0 + a.KW; ++w)
#pragma unroll
                            for (int h = 0; h < 4; ++h) osum += red[(w * 4 + h) * 16 + onn];
                    } else {
                        for (int w = w0; w < w0 + a.KW; ++w) osum += red[(w * 8 + omm) * 16 + onn];
                    }
                    if (a.S == 1) {
                        if (ot * TILE_ROWS + onn < a.n)
                            a.y[(int64_t)omm * a.n + ot * TILE_ROWS + onn] = sm.sx[omm] * osum;
                    } else {
                        const u64 v = ((u64)sm.tag << 32) | __float_as_uint(osum);
                        __hip_atomic_store(&a.part[((ot * a.S + s) * M + omm) * 16 + onn], v,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[rr] = 0.0f;
        }
    };

    for (int base = 0; base < iters; base += PIPE) {
#pragma unroll
        for (int d = 0; d < PIPE; ++d) {
            const int i = base + d;
            process(i, wbuf[d], hbuf[d], sbuf[d]);
            load(i + PIPE, wbuf[d], hbuf[d], sbuf[d]);
        }
    }

    // 5. merge the slices' partials: the last workgroup of each tile adds them
    if (a.S > 1) {
        __syncthreads();
        for (int c0 = 0; c0 < ntile; c0 += kMaxTilesPerGroup) {
            const int nc = min(kMaxTilesPerGroup, ntile - c0);
            if (tid < nc) {
                const int64_t tt = t_begin + c0 + tid;
                const uint32_t old =
                    __hip_atomic_fetch_add(&a.cnt[tt], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int lst = (old == (uint32_t)(a.S - 1));
                if (lst) __hip_atomic_store(&a.cnt[tt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sm.last[tid] = lst;
            }
            __syncthreads();
            for (int e = tid; e < nc * M * 16; e += NT) {
                const int ci = e / (M * 16);
                if (!sm.last[ci]) continue;
                const int omm = (e / 16) % M;
                const int onn = e & 15;
                const int64_t ot = t_begin + c0 + ci;
                float tot = 0.0f;
                for (int sl = 0; sl < a.S; ++sl) {
                    // Every partial was stored before its workgroup counted the tile, so its
                    // tag shows up shortly; the bound only guards against a hang (a missing
                    // partial would turn y into NaN rather than stall the GPU).
                    const u64* p = &a.part[((ot * a.S + sl) * M + omm) * 16 + onn];
                    u64 v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    for (int it = 0; (uint32_t)(v >> 32) != sm.tag && it < (1 << 24); ++it)
                        v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    tot += ((uint32_t)(v >> 32) == sm.tag) ? __uint_as_float((uint32_t)v) : __builtin_nanf("");
                }
                if (ot * TILE_ROWS + onn < a.n) a.y[(int64_t)omm * a.n + ot * TILE_ROWS + onn] = sm.sx[omm] * tot;
            }
            __syncthreads();
        }
        // generation bookkeeping for the exchange words and tags
        if (tid == 0) {
            const uint32_t old =
                __hip_atomic_fetch_add(&a.ws->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old == (uint32_t)(a.P - 1)) {
                __hip_atomic_store(&a.ws->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&a.ws->gen, sm.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// --------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------

typedef void (*KernelFn)(KArgs);

template <int FMT, int PRO, int XT, int GS>
KernelFn pick_dot(bool dot4) {
    return dot4 ? gemm_kernel<FMT, PRO, XT, GS, true> : gemm_kernel<FMT, PRO, XT, GS, false>;
}
template <int FMT, int PRO, int XT>
KernelFn pick_gs(int gs, bool dot4) {
    switch (gs) {
        case 1: return pick_dot<FMT, PRO, XT, 1>(dot4);
        case 2: return pick_dot<FMT, PRO, XT, 2>(dot4);
        default: return pick_dot<FMT, PRO, XT, 4>(dot4);
    }
}
template <int FMT, int PRO>
KernelFn pick_xt(int xt, int gs, bool dot4) {
    return xt == 1 ? pick_gs<FMT, PRO, 1>(gs, dot4) : pick_gs<FMT, PRO, 0>(gs, dot4);
}
template <int FMT>
KernelFn pick_pro(int pro, int xt, int gs, bool dot4) {
    switch (pro) {
        case PRO_RMSNORM: return pick_xt<FMT, PRO_RMSNORM>(xt, gs, dot4);
        case PRO_SWIGLU: return pick_xt<FMT, PRO_SWIGLU>(xt, gs, dot4);
        default: return pick_xt<FMT, PRO_NONE>(xt, gs, dot4);
    }
}
KernelFn pick(int fmt, int pro, int xt, int gs, bool dot4) {
    return fmt == FMT_W6 ? pick_pro<FMT_W6>(pro, xt, gs, dot4) : pick_pro<FMT_W4>(pro, xt, gs, dot4);
}

struct DevState {
    int cus = 0;
    void* ws = nullptr;      // [WsHeader][cnt: cap_t uint32][part: cap_part u64]
    int64_t cap_t = 0;
    size_t cap_part = 0;
};
std::mutex g_mu;
DevState g_dev[64];

int g_split_override = 0;

}  // namespace

// ---------------------------------------------------------------------------
// launch planning (pure host logic)
// ---------------------------------------------------------------------------

Plan make_plan(const Geom& G, int m, int pro, int cus, int split_override) {
    Plan p;
    (void)pro;
    const int KB = (int)G.KB;
    const int T = (int)G.T;
    const bool dot4 = (m == 1);
    p.WPR = NW / m;                               // waves per activation row
    const int tpr = p.WPR * 64;
    auto fits = [&](int s) { return (G.k / s) / 8 <= (int64_t)tpr * MO; };
    auto lds_of = [&](int s) {
        const size_t KS = (size_t)(G.k / s);
        const size_t qs = dot4 ? (KS / 8) * 4 : (KS / G.g) * 8 * 4;
        return (size_t)m * (KS + 32) + qs + 2 * (size_t)NW * 128 * 4;
    };
    const size_t kLdsMax = 150 * 1024;
    int S = 1;
    if (split_override > 0) {
        S = split_override;
    } else {
        // the smallest divisor of KB whose slice fits the thread layout and LDS, and
        // for M > 1 keeps each workgroup's quantisation work (M x K/S) small
        const int64_t want = (m == 1) ? ((int64_t)1 << 40) : 12288;
        for (S = 1; S < SMAX; ++S) {
            if (KB % S != 0) continue;
            if (fits(S) && lds_of(S) <= kLdsMax && (int64_t)m * (G.k / S) <= want) break;
        }
        while (S > 1 && KB % S != 0) --S;
    }
    p.S = S;
    p.KBs = (S > 0 && KB % S == 0) ? KB / S : 0;
    p.KS = (S > 0) ? (int)(G.k / S) : 0;
    int R = (S > 0) ? cus / S : 1;
    if (R > T) R = T;
    if (R < 1) R = 1;
    p.R = R;
    // waves: TW tile groups x KW waves along k (KW divides the slice's
    // super-blocks); with S > 1 one wave is reserved for the exchange
    const int nwa = (S > 1) ? NW - 1 : NW;
    const int tiles_per_wg = (T + R - 1) / R;
    p.KW = 1;
    p.TW = 1;
    int best = -1;
    for (int kw = 1; kw <= nwa && p.KBs > 0; ++kw) {
        if (p.KBs % kw != 0) continue;
        int tw = nwa / kw;
        while (tw > 1 && tw * m * 16 > NT) --tw;      // the epilogue uses one thread per output
        const int used = kw * (tw < tiles_per_wg ? tw : tiles_per_wg);
        if (used > best) {                           // ties: fewer, longer tile flushes
            best = used;
            p.KW = kw;
            p.TW = tw;
        }
    }
    p.spw = p.KW > 0 ? p.KBs / p.KW : 0;
    p.P = S * R;
    p.ks = p.KS + 32;
    p.lds = (S > 0) ? lds_of(S) : 0;
    p.part_floats = (S > 1) ? (size_t)T * S * m * 16 : 0;
    p.ok = S >= 1 && S <= SMAX && KB % S == 0 && p.KBs >= 1 && fits(S) && p.spw >= 1 &&
           p.lds <= kLdsMax && p.P >= 1 && m >= 1 && m <= 8;
    return p;
}

void set_split_override(int s) { g_split_override = s; }

bool gemm_plan_ok(const Geom& G, int m, int pro) {
    return make_plan(G, m, pro, 256, g_split_override).ok;
}

hipError_t launch_gemm(const Geom& G, const GemmCall& c, hipStream_t st) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    DevState& ds = g_dev[dev];
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (ds.cus == 0) {
            int v = 0;
            e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
            if (e != hipSuccess) return e;
            ds.cus = v > 0 ? v : 256;
        }
    }
    const Plan p = make_plan(G, c.m, c.prologue, ds.cus, g_split_override);
    if (!p.ok) return hipErrorInvalidValue;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!ds.ws || ds.cap_t < G.T || ds.cap_part < p.part_floats) {
            int64_t cap_t = ds.cap_t > G.T ? ds.cap_t : G.T;
            if (cap_t < 4096) cap_t = 4096;
            size_t cap_part = ds.cap_part > p.part_floats ? ds.cap_part : p.part_floats;
            if (ds.ws) {
                e = hipDeviceSynchronize();
                if (e != hipSuccess) return e;
                (void)hipFree(ds.ws);
                ds.ws = nullptr;
            }
            const size_t bytes = sizeof(WsHeader) + (size_t)cap_t * 4 + cap_part * 8;
            e = hipMalloc(&ds.ws, bytes);
            if (e != hipSuccess) return e;
            e = hipMemset(ds.ws, 0, bytes);
            if (e != hipSuccess) return e;
            e = hipDeviceSynchronize();
            if (e != hipSuccess) return e;
            ds.cap_t = cap_t;
            ds.cap_part = cap_part;
        }
    }

    const bool dot4 = (c.m == 1);
    const int gs = (int)(G.g / 32);
    KernelFn fn = pick(G.fmt, c.prologue, c.xt, gs, dot4);

    KArgs a;
    a.data = c.data;
    a.x = c.x;
    a.x2 = c.x2;
    a.ld = c.ld;
    a.gamma = c.gamma;
    a.eps = c.eps;
    a.y = c.y;
    a.q_out = c.q_out;
    a.sx_out = c.sx_out;
    a.p_out = c.p_out;
    a.ws = static_cast<WsHeader*>(ds.ws);
    a.cnt = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ds.ws) + sizeof(WsHeader));
    a.part = reinterpret_cast<u64*>(a.cnt + ds.cap_t);
    a.n = (int)G.n;
    a.k = (int)G.k;
    a.m = c.m;
    a.T = (int)G.T;
    a.KB = (int)G.KB;
    a.kg = (int)G.kg;
    a.sb_row = (int)G.sb_row;
    a.wsb_row = (int)G.wsb_row;
    a.tile_full = G.tile_full;
    a.S = p.S;
    a.R = p.R;
    a.P = p.P;
    a.TW = p.TW;
    a.KW = p.KW;
    a.spw = p.spw;
    a.KBs = p.KBs;
    a.KS = p.KS;
    a.WPR = p.WPR;
    a.ks = p.ks;
    a.spin_limit = c.spin_limit > 0 ? c.spin_limit : (1 << 20);

    if (p.lds > 64 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)p.P), dim3(NT), p.lds, st, a);
    return hipGetLastError();
}

}  // namespace sk
