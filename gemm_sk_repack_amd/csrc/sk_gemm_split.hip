// sk_gemm_split.hip -- the split path kept for comparison: GEMM kernels that
// read 4-bit weights straight from the canonical [codes | scales] layout, with
// the activations quantised in the launch or by a separate kernel, and that
// separate quantisation kernel.
#include "sk_gemm_kernel.h"

namespace sk {

KernelFn pick_kernel_split(int pro, int xt, int gs, bool dot4, bool wide) {
    if (pro == PRO_QIN) return pick_canon_gs<PRO_QIN, 0>(gs, dot4, false);
    return xt == 1 ? pick_canon_gs<PRO_NONE, 1>(gs, dot4, wide) : pick_canon_gs<PRO_NONE, 0>(gs, dot4, wide);
}

}  // namespace sk

namespace sk {
namespace {

// One workgroup per activation row: the row's absmax, then sx = absmax/127 and
// q = rint(h/sx) with the same arithmetic as the GEMM's in-launch quantiser
// (two products that bracket fp32(h/sx); exact division where they round to
// different integers), written to memory.
constexpr int QT = 256;
template <int XT>
__global__ __launch_bounds__(QT) void quantize_kernel(const void* x, int k, int8_t* q, float* sx_out) {
    constexpr int E = XT == 0 ? 4 : 8;              // elements per 16-byte chunk
    __shared__ float wmax[QT / 64];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const uint8_t* row = static_cast<const uint8_t*>(x) + (int64_t)m * k * (XT == 0 ? 4 : 2);
    const int nch = k / E;
    auto chunk = [&](const int c, float v[E]) {
        const uint4 raw = *reinterpret_cast<const uint4*>(row + (int64_t)c * 16);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[e] = XT == 0 ? __uint_as_float(w[e])
                           : __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
    };
    float mx = 0.0f;
    for (int c = tid; c < nch; c += QT) {
        float v[E];
        chunk(c, v);
#pragma unroll
        for (int e = 0; e < E; ++e) mx = fmaxf(mx, fabsf(v[e]));
    }
    mx = wave_max(mx);
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    float amx = 0.0f;
#pragma unroll
    for (int w = 0; w < QT / 64; ++w) amx = fmaxf(amx, wmax[w]);
    const float sx = (amx > 0.0f) ? amx / 127.0f : 0.0f;
    const float inv = (sx > 0.0f) ? 1.0f / sx : 0.0f;   // sx == 0: every code is 0
    const float inv_lo = inv * kInvLo, inv_hi = inv * kInvHi;
    if (tid == 0) sx_out[m] = sx;
    for (int c = tid; c < nch; c += QT) {
        float v[E];
        chunk(c, v);
        uint32_t b[E];
        uint32_t split = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) b[e] = code_bits(v[e], inv_lo, inv_hi, split);
        if (sx < kMinCorrectedSx && sx > 0.0f) {
#pragma unroll
            for (int e = 0; e < E; ++e) b[e] = __float_as_uint(v[e] / sx + kRoundMagic);
        } else if (split != 0) {
#pragma unroll
            for (int e = 0; e < E; ++e) b[e] = corrected_code_bits(v[e], sx, inv);
        }
        int8_t* dst = q + (int64_t)m * k + (int64_t)c * E;
        if constexpr (E == 4) {
            *reinterpret_cast<uint32_t*>(dst) = pack_low_bytes(b[0], b[1], b[2], b[3]);
        } else {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_low_bytes(b[0], b[1], b[2], b[3]),
                                                        pack_low_bytes(b[4], b[5], b[6], b[7]));
        }
    }
}

// The split path's prologues: h = RMSNorm(x) (one workgroup per activation
// row, which reduces it) or h = SwiGLU(gate, up) (elementwise, QT chunks per
// workgroup) written to memory as float32, with the fused
// prologue's arithmetic (the sum of squares in float64, then the correctly
// rounded fp32 sqrt and reciprocal, then two rounded products; silu through
// sk_expf).
template <int PRO, int XT>
__global__ __launch_bounds__(QT) void prologue_kernel(const void* x, const void* x2, int64_t ld,
                                                      const float* gamma, float eps, int k, float* h) {
    constexpr int E = XT == 0 ? 4 : 8;              // elements per 16-byte chunk
    __shared__ double wsum[QT / 64];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t rs = ld * (XT == 0 ? 4 : 2);      // row stride in bytes
    const uint8_t* row = static_cast<const uint8_t*>(x) + (int64_t)m * rs;
    const uint8_t* row2 = PRO == PRO_SWIGLU ? static_cast<const uint8_t*>(x2) + (int64_t)m * rs : row;
    float* out = h + (int64_t)m * k;
    const int nch = k / E;
    auto chunk = [&](const uint8_t* base, const int c, float v[E]) {
        const uint4 raw = *reinterpret_cast<const uint4*>(base + (int64_t)c * 16);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[e] = XT == 0 ? __uint_as_float(w[e])
                           : __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
    };
    auto store = [&](const int c, const float o[E]) {
#pragma unroll
        for (int e = 0; e < E; e += 4)
            *reinterpret_cast<float4*>(out + (int64_t)c * E + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
    };
    if constexpr (PRO == PRO_SWIGLU) {
        // elementwise: workgroup (m, j) takes chunks [j * QT, (j + 1) * QT) of the row
        for (int c = blockIdx.y * QT + tid; c < nch && c < (int)(blockIdx.y + 1) * QT; c += QT) {
            float g[E], u[E], o[E];
            chunk(row, c, g);
            chunk(row2, c, u);
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = silu_mul(g[e], u[e]);
            store(c, o);
        }
    } else {
        double ss = 0.0;
        for (int c = tid; c < nch; c += QT) {
            float v[E];
            chunk(row, c, v);
#pragma unroll
            for (int e = 0; e < E; ++e) ss += (double)v[e] * (double)v[e];
        }
        ss = wave_sum(ss);
        if ((tid & 63) == 0) wsum[tid >> 6] = ss;
        __syncthreads();
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < QT / 64; ++w) tot += wsum[w];
        const float ms = (float)(tot / (double)k);
        const float d = ms + eps;
        const float sd = (float)__builtin_sqrt((double)d);   // correctly rounded fp32 sqrt
        const float rr = (float)(1.0 / (double)sd);          // correctly rounded fp32 1/x
        for (int c = tid; c < nch; c += QT) {
            float v[E], o[E];
            chunk(row, c, v);
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                const float4 gv = *reinterpret_cast<const float4*>(gamma + (int64_t)c * E + e);
                o[e] = rms_apply(v[e], rr, gv.x);
                o[e + 1] = rms_apply(v[e + 1], rr, gv.y);
                o[e + 2] = rms_apply(v[e + 2], rr, gv.z);
                o[e + 3] = rms_apply(v[e + 3], rr, gv.w);
            }
            store(c, o);
        }
    }
}

}  // namespace

hipError_t launch_prologue(int pro, const void* x, const void* x2, int64_t ld, int xt, const float* gamma,
                           float eps, int m, int64_t k, float* h, hipStream_t st) {
    if (pro == PRO_SWIGLU) {
        const unsigned nblk = (unsigned)((k / (xt == 1 ? 8 : 4) + QT - 1) / QT);   // chunk blocks per row
        if (xt == 1) hipLaunchKernelGGL((prologue_kernel<PRO_SWIGLU, 1>), dim3(m, nblk), dim3(QT), 0, st, x, x2, ld, gamma, eps, (int)k, h);
        else hipLaunchKernelGGL((prologue_kernel<PRO_SWIGLU, 0>), dim3(m, nblk), dim3(QT), 0, st, x, x2, ld, gamma, eps, (int)k, h);
    } else {
        if (xt == 1) hipLaunchKernelGGL((prologue_kernel<PRO_RMSNORM, 1>), dim3(m), dim3(QT), 0, st, x, x2, ld, gamma, eps, (int)k, h);
        else hipLaunchKernelGGL((prologue_kernel<PRO_RMSNORM, 0>), dim3(m), dim3(QT), 0, st, x, x2, ld, gamma, eps, (int)k, h);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int xt, int m, int64_t k, int8_t* q, float* sx,
                           hipStream_t st) {
    if (xt == 1) hipLaunchKernelGGL(quantize_kernel<1>, dim3(m), dim3(QT), 0, st, x, (int)k, q, sx);
    else hipLaunchKernelGGL(quantize_kernel<0>, dim3(m), dim3(QT), 0, st, x, (int)k, q, sx);
    return hipGetLastError();
}

}  // namespace sk
