// sk_gemm.hip -- skinny quantized GEMM kernels for gfx950 (MI355X).
//
//   y[m][n] = sx[m] * sum_j s[n][j] * P[m][n][j],   m < M <= 8,
//   P[m][n][j] = sum_{k in group j} w[n][k] * q[m][k]          (exact int32)
//
// ("Doubling the LLM token rate in ComfyUI", section on optimizing linear
// kernels; "Comfy quantization formats", sections on weight formats and on
// activations.)  One launch does everything:
//
//  1. Each workgroup issues the 128-bit loads of its first super-blocks, then
//     runs the activation prologue while they are in flight: optional RMSNorm
//     or SwiGLU, per-row absmax, sx = absmax/127, q = rint(h/sx) -> int8 in
//     LDS, plus the per-group sums of q used to undo the weights' offset
//     binary encoding (u = w + 8 or w + 32, so P = sum u*q - off*sum q).
//  2. Waves stream their contiguous share of each 16-row tile.  M >= 2 uses
//     v_mfma_i32_16x16x32_i8 with q as the A operand (M padded to 16) and the
//     unpacked weights as B; M = 1 uses v_dot4_i32_i8.  The offset correction
//     is the accumulator's initial value, so the integer result is the exact
//     per-group partial; it is scaled by the group's FP32 scale and
//     accumulated in fp32.
//  3. Per tile, the waves' partial sums are added in a fixed order through LDS
//     and y is written.  No atomics on the output: results are deterministic.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sk_internal.h"

namespace sk {

namespace {

constexpr int NW = 8;          // waves per workgroup
constexpr int NT = NW * 64;    // threads per workgroup
constexpr int PIPE = 4;        // super-blocks in flight per wave

typedef int v4i __attribute__((ext_vector_type(4)));

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
    int n, k, m;
    int T, KB, kg;
    int sb_row, wsb_row;
    int64_t tile_full;
    int P;     // workgroups in the grid
    int spw;   // super-block slots per wave per tile
    int ks;    // LDS row stride of q in bytes
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

// h for 8 consecutive elements of row m starting at column k0
template <int PRO, int XT>
__device__ inline void prologue8(const KArgs& a, int m, int k0, float r_m, float v[8]) {
    if (PRO == PRO_SWIGLU) {
        float g[8], u[8];
        load8<XT>(a.x, (int64_t)m * a.ld + k0, g);
        load8<XT>(a.x2, (int64_t)m * a.ld + k0, u);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float den = 1.0f + sk_expf(-g[e]);
            float silu = g[e] / den;
            v[e] = silu * u[e];
        }
    } else {
        load8<XT>(a.x, (int64_t)m * a.ld + k0, v);
        if (PRO == PRO_RMSNORM) {
            const float4* gp = reinterpret_cast<const float4*>(a.gamma + k0);
            float4 g0 = gp[0], g1 = gp[1];
            float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float t = v[e] * r_m;
                v[e] = t * gm[e];
            }
        }
    }
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

// --------------------------------------------------------------------------
// the kernel
// --------------------------------------------------------------------------

template <int FMT, int PRO, int XT, int GS, bool DOT4>
__global__ __launch_bounds__(NT) void gemm_kernel(KArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int NG = 4 / GS;                  // groups per super-block
    constexpr int OFF = (FMT == FMT_W6) ? 32 : 8;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int nl = lane & 15;                   // B column (row n of the tile) / A row (m)
    const int hl = lane >> 4;                   // k-octet within a 32-k block
    const int M = a.m;
    const int K = a.k;
    const int K8 = K >> 3;

    // LDS carve-up
    int8_t* q_l = reinterpret_cast<int8_t*>(lds);                               // [M][ks]
    int32_t* qs_l = reinterpret_cast<int32_t*>(lds + (size_t)M * a.ks);          // sums of q
    const int qs_n = DOT4 ? K8 : a.kg * 8;                                       // octet sums | [kg][8]
    float* red_l = reinterpret_cast<float*>(qs_l + qs_n);                        // [NW][8][16]
    float* sx_l = red_l + NW * 128;                                              // [8]
    float* fst_l = sx_l + 8;                                                     // [NW][8]
    double* dst_l = reinterpret_cast<double*>(fst_l + NW * 8);                  // [NW][8]

    const int64_t t_begin = (int64_t)blockIdx.x * a.T / a.P;
    const int64_t t_end = (int64_t)(blockIdx.x + 1) * a.T / a.P;
    const int total = (int)(t_end - t_begin) * a.spw;

    uint4 wbuf[PIPE];
    uint2 hbuf[PIPE];
    float sbuf[PIPE][NG];

    auto load = [&](int i, uint4& w4, uint2& h2, float* s) {
        w4 = make_uint4(0u, 0u, 0u, 0u);
        h2 = make_uint2(0u, 0u);
#pragma unroll
        for (int g = 0; g < NG; ++g) s[g] = 0.0f;
        if (i >= total) return;
        const int64_t t = t_begin + i / a.spw;
        const int kb = wv * a.spw + i % a.spw;
        if (kb >= a.KB) return;
        const int64_t rem = (int64_t)a.n - t * TILE_ROWS;
        const int nr = rem < TILE_ROWS ? (int)rem : TILE_ROWS;
        if (nl >= nr) return;
        const uint8_t* tb = a.data + t * a.tile_full;
        const uint8_t* wp = tb + (nr == TILE_ROWS ? (int64_t)kb * nr * a.sb_row
                                                   : (int64_t)kb * nr * a.wsb_row);
        const uint8_t* sp = tb + (nr == TILE_ROWS ? (int64_t)kb * nr * a.sb_row + nr * a.wsb_row
                                                   : (int64_t)a.KB * nr * a.wsb_row +
                                                         (int64_t)kb * nr * NG * 4);
        w4 = *reinterpret_cast<const uint4*>(wp + (hl * nr + nl) * 16);
        if (FMT == FMT_W6) h2 = *reinterpret_cast<const uint2*>(wp + nr * 64 + (hl * nr + nl) * 8);
        const float* sf = reinterpret_cast<const float*>(sp) + nl * NG;
        if (NG == 4) {
            float4 v = *reinterpret_cast<const float4*>(sf);
            s[0] = v.x; s[1] = v.y; s[2 % NG] = v.z; s[3 % NG] = v.w;
        } else if (NG == 2) {
            float2 v = *reinterpret_cast<const float2*>(sf);
            s[0] = v.x; s[1 % NG] = v.y;
        } else {
            s[0] = sf[0];
        }
    };

    // 1a. prime the weight stream
#pragma unroll
    for (int d = 0; d < PIPE; ++d) load(d, wbuf[d], hbuf[d], sbuf[d]);

    // 1b. activation prologue
    for (int i = tid; i < qs_n; i += NT) qs_l[i] = 0;

    float rr[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) rr[m] = 1.0f;
    if (PRO == PRO_RMSNORM) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if (m < M) {
                double ss = 0.0;
                for (int o = tid; o < K8; o += NT) {
                    float v[8];
                    load8<XT>(a.x, (int64_t)m * a.ld + 8 * o, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss += (double)v[e] * (double)v[e];
                }
                ss = wave_sum(ss);
                if (lane == 0) dst_l[wv * 8 + m] = ss;
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if (m < M) {
                double ss = 0.0;
                for (int w = 0; w < NW; ++w) ss += dst_l[w * 8 + m];
                float ms = (float)(ss / (double)K);
                float d = ms + a.eps;
                float sd = (float)__builtin_sqrt((double)d);     // correctly rounded fp32 sqrt
                rr[m] = (float)(1.0 / (double)sd);                 // correctly rounded fp32 1/x
            }
        }
    }
    // absmax of h
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        if (m < M) {
            float mx = 0.0f;
            for (int o = tid; o < K8; o += NT) {
                float v[8];
                prologue8<PRO, XT>(a, m, 8 * o, rr[m], v);
#pragma unroll
                for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
            }
            mx = wave_max(mx);
            if (lane == 0) fst_l[wv * 8 + m] = mx;
        }
    }
    __syncthreads();
    if (tid < 8) {
        float mx = 0.0f;
        if (tid < M)
            for (int w = 0; w < NW; ++w) mx = fmaxf(mx, fst_l[w * 8 + tid]);
        float sx = mx / 127.0f;
        sx_l[tid] = (mx > 0.0f) ? sx : 0.0f;
        if (a.sx_out && blockIdx.x == 0 && tid < M) a.sx_out[tid] = sx_l[tid];
    }
    __syncthreads();
    // quantise into LDS
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        if (m < M) {
            const float sx = sx_l[m];
            for (int o = tid; o < K8; o += NT) {
                float v[8];
                prologue8<PRO, XT>(a, m, 8 * o, rr[m], v);
                uint32_t lo = 0, hi = 0;
                int sum = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    int qi = 0;
                    if (sx > 0.0f) {
                        float t = v[e] / sx;
                        t = __builtin_rintf(t);
                        t = fminf(fmaxf(t, -127.0f), 127.0f);
                        qi = (int)t;
                    }
                    sum += qi;
                    uint32_t b = (uint32_t)(qi & 0xFF);
                    if (e < 4) lo |= b << (8 * e); else hi |= b << (8 * (e - 4));
                }
                *reinterpret_cast<uint2*>(q_l + m * a.ks + 8 * o) = make_uint2(lo, hi);
                if (a.q_out && blockIdx.x == 0)
                    *reinterpret_cast<uint2*>(a.q_out + (int64_t)m * K + 8 * o) = make_uint2(lo, hi);
                if (DOT4) qs_l[o] = sum;
                else atomicAdd(&qs_l[(8 * o / (32 * GS)) * 8 + m], sum);
            }
        }
    }
    __syncthreads();

    // 2. stream the weights
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int ml = nl;   // A-operand row (activation row m) of this lane

    for (int base = 0; base < total; base += PIPE) {
#pragma unroll
        for (int d = 0; d < PIPE; ++d) {
            const int i = base + d;
            if (i < total) {
                const int64_t t = t_begin + i / a.spw;
                const int slot = i % a.spw;
                const int kb = wv * a.spw + slot;
                const int64_t rem = (int64_t)a.n - t * TILE_ROWS;
                const int nr = rem < TILE_ROWS ? (int)rem : TILE_ROWS;
                if (kb < a.KB) {
                    uint32_t wd[4] = {wbuf[d].x, wbuf[d].y, wbuf[d].z, wbuf[d].w};
                    uint32_t lo[4], hi[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        lo[j] = wd[j] & 0x0F0F0F0Fu;
                        hi[j] = (wd[j] >> 4) & 0x0F0F0F0Fu;
                        if (FMT == FMT_W6) {
                            const uint32_t hd = (j < 2) ? hbuf[d].x : hbuf[d].y;
                            if ((j & 1) == 0) {
                                lo[j] |= (hd << 4) & 0x30303030u;
                                hi[j] |= (hd << 2) & 0x30303030u;
                            } else {
                                lo[j] |= hd & 0x30303030u;
                                hi[j] |= (hd >> 2) & 0x30303030u;
                            }
                        }
                    }
                    const int kbase = kb * 128;
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
                            acc[0] = __builtin_fmaf(sbuf[d][gi], (float)pg, acc[0]);
                            if (a.p_out && nl < nr)
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
                            const int gg = kb * NG + gi;
                            v4i c = {0, 0, 0, 0};
                            if (hl < 2) {
                                const int4 qv = *reinterpret_cast<const int4*>(qs_l + gg * 8 + 4 * hl);
                                c[0] = -OFF * qv.x; c[1] = -OFF * qv.y;
                                c[2] = -OFF * qv.z; c[3] = -OFF * qv.w;
                            }
#pragma unroll
                            for (int jj = 0; jj < GS; ++jj)
                                c = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[gi * GS + jj],
                                                                         bv[gi * GS + jj], c, 0, 0, 0);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                acc[r] = __builtin_fmaf(sbuf[d][gi], (float)c[r], acc[r]);
                                const int mm = 4 * hl + r;
                                if (a.p_out && mm < M && nl < nr)
                                    a.p_out[((int64_t)mm * a.n + t * TILE_ROWS + nl) * a.kg + gg] = c[r];
                            }
                        }
                    }
                }
                load(i + PIPE, wbuf[d], hbuf[d], sbuf[d]);

                if (slot == a.spw - 1) {
                    // 3. tile epilogue: fixed-order sum of the waves' partials
                    if (DOT4) {
                        red_l[(wv * 4 + hl) * 16 + nl] = acc[0];
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int mm = 4 * hl + r;
                            if (mm < M) red_l[(wv * 8 + mm) * 16 + nl] = acc[r];
                        }
                    }
                    __syncthreads();
                    if (tid < M * 16) {
                        const int mm = tid >> 4, nn = tid & 15;
                        float s = 0.0f;
                        if (DOT4) {
                            for (int w = 0; w < NW; ++w)
#pragma unroll
                                for (int h = 0; h < 4; ++h) s += red_l[(w * 4 + h) * 16 + nn];
                        } else {
                            for (int w = 0; w < NW; ++w) s += red_l[(w * 8 + mm) * 16 + nn];
                        }
                        if (nn < nr) a.y[(int64_t)mm * a.n + t * TILE_ROWS + nn] = sx_l[mm] * s;
                    }
                    __syncthreads();
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] = 0.0f;
                }
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

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

}  // namespace

size_t gemm_lds_bytes(const Geom& G, int m) {
    const bool dot4 = (m == 1);
    size_t ks = (size_t)G.k + 32;
    size_t qs = dot4 ? (size_t)(G.k / 8) * 4 : (size_t)G.kg * 8 * 4;
    return (size_t)m * ks + qs + NW * 128 * 4 + 8 * 4 + NW * 8 * 4 + NW * 8 * 8;
}

hipError_t launch_gemm(const Geom& G, const GemmCall& c, hipStream_t st) {
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
    a.n = (int)G.n;
    a.k = (int)G.k;
    a.m = c.m;
    a.T = (int)G.T;
    a.KB = (int)G.KB;
    a.kg = (int)G.kg;
    a.sb_row = (int)G.sb_row;
    a.wsb_row = (int)G.wsb_row;
    a.tile_full = G.tile_full;
    a.ks = (int)G.k + 32;
    a.spw = (int)((G.KB + NW - 1) / NW);
    int64_t P = 2 * (int64_t)device_cus();
    if (P > G.T) P = G.T;
    a.P = (int)P;

    const size_t lds = gemm_lds_bytes(G, c.m);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)P), dim3(NT), lds, st, a);
    return hipGetLastError();
}

}  // namespace sk
