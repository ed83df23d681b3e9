// sk_gemm_kernel.h -- the skinny quantized GEMM kernel for gfx950 (MI355X).
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
//  1. Load this thread's activations first (they head the longest chain:
//     x -> statistics -> q -> every dot product), then the first PRIME
//     super-blocks of the weight stream.  Every load is unconditional (an
//     out-of-range slot reads a harmless in-bounds address), so the number of
//     outstanding loads is known at compile time and waiting for the
//     activations never waits for the weight stream.
//  2. Activation prologue while the weights are in flight: optional RMSNorm or
//     SwiGLU; per-row statistics.  With S > 1 the full-row sum of squares and
//     absmax are exchanged between slices through tagged device-scope words
//     (one wave publishes and polls; the wait is bounded and a time-out falls
//     back to computing the missing slices locally).  Then sx = absmax/127 and
//     q = rint(h/sx) -> int8 in LDS.  This code runs once per launch, so it is
//     kept short and straight: every instruction of it is a cold fetch.
//  3. Stream the tiles through a register pipeline of PIPE slots.  Weight
//     codes are two's complement; the bytes fed to the dot products hold
//     w << 4 (W4) or w << 2 (W6), so the integer sums are the exact per-group
//     partials times 16 or 4 (undone by a power of two at the store).  M >= 2
//     uses v_mfma_i32_16x16x32_i8 (q = A operand, M padded to 16; weights =
//     B); M = 1 uses v_dot4_i32_i8.  Each partial is scaled by its FP32 group
//     scale and accumulated in fp32.
//  4. Per tile, the waves' sums are added in a fixed order through LDS.  With
//     S = 1 the workgroup writes y.  Otherwise it stores a tagged partial; at
//     the end, the last of a tile's S workgroups to arrive adds the S
//     partials in slice order and writes y.  No floating-point atomics and no
//     cache-flushing fences: results are deterministic.
//
// Included by one translation unit per weight format and build flavour, each
// instantiating its kernels (sk_gemm_*.hip); the launch logic is in sk_gemm.hip.
#ifndef SK_GEMM_KERNEL_H
#define SK_GEMM_KERNEL_H

#include <hip/hip_runtime.h>

#include "sk_internal.h"

namespace sk {


constexpr int NW = 16;         // waves per workgroup
constexpr int NT = NW * 64;    // threads per workgroup
// Register pipeline of the weight stream: super-blocks in flight per wave, and
// how many of them each wave issues before the activation prologue, for the
// v_dot4 instances (M = 1) and the MFMA instances (M >= 2, the codebook).
#ifndef SK_PIPE_DOT4
#define SK_PIPE_DOT4 5
#endif
#ifndef SK_PRIME_DOT4
#define SK_PRIME_DOT4 2
#endif
#ifndef SK_PIPE_MFMA
#define SK_PIPE_MFMA 5
#endif
#ifndef SK_PRIME_MFMA
#define SK_PRIME_MFMA 2
#endif
// M >= 2: a wave's first weight loads wait for its own activations (2), for
// every wave's (1, a workgroup barrier), or go out at once (0)
#ifndef SK_MFMA_ACT_FIRST
#define SK_MFMA_ACT_FIRST 2
#endif
// G = 32 scales on the v_dot4 path: one per lane (1), or the row's four (0)
#ifndef SK_SCALE1
#define SK_SCALE1 1
#endif
// The rest of the first load group issued one slot per quantised chunk (1: on
// the MFMA path, 2: on the v_dot4 path too), or all of it after the quantiser (0)
#ifndef SK_REST_IN_Q
#define SK_REST_IN_Q 1
#endif
constexpr int kPipeDot4 = SK_PIPE_DOT4, kPrimeDot4 = SK_PRIME_DOT4;
constexpr int kPipeMfma = SK_PIPE_MFMA, kPrimeMfma = SK_PRIME_MFMA;
// The codebook keeps 4 (its G = 16 scales take two registers more per slot).
constexpr int kPipeCb = 4;
constexpr int pipe_of(bool dot4, bool cb) { return cb ? kPipeCb : dot4 ? kPipeDot4 : kPipeMfma; }
constexpr int SMAX = 32;       // largest number of K-slices
// Tile-epilogue LDS: per half, [tile group][row][column][kwp] floats, kwp =
// the k-parts per tile group rounded up to 4, 8 or 16 (the entries past KW
// stay zero), so a thread sums its output's partials without masks.
constexpr int red_kwp(int kw) { return kw <= 4 ? 4 : kw <= 8 ? 8 : 16; }
// Weight-stream buffer loads: the resource of a slot group spans kRsrcMax bytes
// from the group's first byte (every real slot lies inside), and an offset of
// kOutside lies past it, so such a load returns zeros without touching memory.
constexpr int kRsrcMax = 0x7FFFFFFF;
constexpr int kOutside = (int)0x80000000u;
constexpr int kRsrcFlags = 0x00020000;   // raw (untyped) 32-bit dword access
#ifndef SK_STREAM_POLICY
#define SK_STREAM_POLICY 18
#endif
// Cache policy of the weight stream: non-temporal (2) at device scope (16).
// Each weight byte is read once per call; on a streaming probe of the decoder
// and lm_head sizes this policy read 10-17% faster than the default one.
constexpr int kStreamPolicy = SK_STREAM_POLICY;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned long long u64;
struct KArgs {
    // Read at kernel entry, before the first loads: one contiguous block, so
    // every wave fetches it with a few wide scalar loads in one round trip.
    const uint8_t* data;
    const void* x;
    int64_t ld;
    // stream-layout addressing: full tiles (16 rows) and the ragged last tile
    int64_t tile_full;      // bytes per full tile
    int64_t rag_w, rag_s;   // byte offsets of the ragged tile's weights and scales
    int m, KS, S, KBs;
    // tiles of block r: [r * tq + min(r, trem), ... + tq + (r < trem)); jn1 / jn0
    // = tiles per tile group, rounded up, for the two block sizes
    int tq, trem, jn0, jn1;
    int TW, spw, KB;
    int srem;               // super-blocks per wave along k: spw, plus one for the first srem k-parts
    int sbf, swo;           // bytes per super-block of a full tile; offset of its scales
    int t_rag;              // index of the ragged tile, -1 if N % 16 == 0
    int nr_last;            // rows of the ragged tile (16 if none)
    int rag_sbw, rag_sbs;   // its weight and scale bytes per super-block
    int cpr, tpr;           // activation chunks per row of the slice; threads per row
    // expert banks: logical tile t is tile t % tpe of expert experts[t / tpe]
    // (a device array) in the bank of n_experts experts (tpe = tiles per
    // expert; 0 for a plain weight)
    int tpe;
    // per wave: tile group (bits 0-4), k-part (5-9), activation row (10-13),
    // wave index within the row (14-18) and activation chunk steps (19-22)
    uint32_t wtab[NW];
    // used later in the launch
    int n_experts;
    const int32_t* experts;
    const float* codebook;  // 16 levels (codebook format only)
    const void* x2;
    const float* gamma;
    float eps;
    float* y;
    int8_t* q_out;
    float* sx_out;
    int32_t* p_out;
    WsHeader* ws;           // caller-owned workspace (S > 1 only)
    u64* part;              // its tagged split-K partials
    int n, k;
    int T, kg;
    int R, P, KW, WPR, ks;
    int m_magic;            // (65536 + M - 1) / M: x / M = (x * m_magic) >> 16 for x < 64
    int kwp, red_half;      // partials pitch and floats per half of the tile-epilogue buffer
    u64 tpe_magic;          // floor(2^40 / tpe) + 1: t / tpe = (t * tpe_magic) >> 40 for t < 2^20
    int spin_limit;
};

struct Smem {
    alignas(16) double wd[NW];          // per-wave values
    alignas(16) float wf[NW];
    alignas(16) double exd[8 * SMAX];   // [row][slice] statistics of the slices
    alignas(16) float exf[8 * SMAX];
    float sx[8];
    float inv[8];
    float rr[8];
    int miss[SMAX];
    uint32_t tag;
    int last;
};

typedef void (*KernelFn)(KArgs);

// One picker per (format, debug exports) translation unit.
KernelFn pick_kernel_w4(int pro, int xt, int gs, bool dot4, bool wide);
KernelFn pick_kernel_w6(int pro, int xt, int gs, bool dot4, bool wide);
KernelFn pick_kernel_cb(int pro, int xt, int gs, bool dot4, bool wide);
KernelFn pick_kernel_w4_dbg(int pro, int xt, int gs, bool dot4, bool wide);
KernelFn pick_kernel_w6_dbg(int pro, int xt, int gs, bool dot4, bool wide);
KernelFn pick_kernel_cb_dbg(int pro, int xt, int gs, bool dot4, bool wide);
KernelFn pick_kernel_split(int pro, int xt, int gs, bool dot4, bool wide);
// 4-bit weights, no prologue, production: the instances with a 4-slot pipeline
KernelFn pick_kernel_w4_pipe4(int xt, int gs, bool dot4, bool wide);

namespace {


// --------------------------------------------------------------------------
// activation helpers
// --------------------------------------------------------------------------

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

// Activation codes q = clamp(rint(fp32(h / sx)), -127, 127), packed as int8
// four to a dword.  For sx > 0, |h| <= 127 sx so the clamp never acts.
// fma(h, c, 1.5 * 2^23) with |h c| < 2^22 rounds the exact product h c to the
// nearest integer (ties to even) and leaves it in the low mantissa bits, so the
// low byte of the result's bit pattern is the int8 code.  With inv = fp32(1/sx)
// (correctly rounded), inv_lo = fp32(inv (1 - 2^-22)) and inv_hi =
// fp32(inv (1 + 2^-22)) satisfy inv_lo <= (1 - 2^-24) / sx and inv_hi >=
// (1 + 2^-24) / sx (three relative errors of at most 2^-24 each), and
// fp32(h/sx) is within a factor 1 +- 2^-24 of h/sx, so fp32(h/sx) lies between
// h inv_lo and h inv_hi.  Rounding to the nearest integer is monotone: where the
// two products round to the same integer, fp32(h/sx) rounds to it too.  Where
// they differ (the quotient within about |h/sx| 2^-22 of a half-integer: with
// bf16 activations every element equal to half the row's maximum, 63.5 before
// sx is rounded, is such a case) the quotient itself is formed, by
// corrected_code_bits; a row with a tiny sx takes IEEE division throughout.
constexpr float kRoundMagic = 12582912.0f;   // 1.5 * 2^23
constexpr float kInvLo = 0x1.fffff8p-1f;      // 1 - 2^-22
constexpr float kInvHi = 0x1.000004p+0f;      // 1 + 2^-22
constexpr float kMinCorrectedSx = 0x1p-100f;  // below it, IEEE division for every element
// Chunks with an element whose bracketing products round apart are listed by
// their wave in LDS (the chunk's h values and its position in q) and redone by
// all 64 lanes of the wave, one element each, rather than by a chunk-wide
// branch that every lane of the wave executes whenever one lane needs it.
// A wave lists at most kWaveFix chunks; any more are redone in place.
constexpr int kWaveFix = 16;
constexpr int kFixCap = NW * kWaveFix;
constexpr int kFixStride = 12;                 // floats per entry: up to 8 h values, position
// Code bits of h (its low byte is the int8 code) from the lower product; `split`
// becomes nonzero when the two products round differently.  Both results are
// 1.5 * 2^23 plus an integer of magnitude <= 128, so their low 16 bits differ
// exactly when the integers do; the sum of absolute differences of those bits
// adds less than 2^16 per element and cannot wrap.
__device__ inline uint32_t code_bits(float h, float inv_lo, float inv_hi, uint32_t& split) {
    const uint32_t lo = __float_as_uint(__builtin_fmaf(h, inv_lo, kRoundMagic));
    const uint32_t hi = __float_as_uint(__builtin_fmaf(h, inv_hi, kRoundMagic));
    split = __builtin_amdgcn_sad_u16(lo, hi, split);
    return lo;
}
// Code bits of h from the correctly rounded quotient fp32(h/sx), formed without
// a division: q0 = fp32(h inv) is within two ulps of h/sx; one correction
// q1 = fp32(q0 + r0 inv), r0 = fp32(h - sx q0) by an FMA, leaves it within one
// ulp; for such a q1 the residual r1 = h - sx q1 is exact in fp32 and, inv being
// the correctly rounded reciprocal, fp32(q1 + r1 inv) is the correctly rounded
// quotient (Markstein's theorem on FMA division).  That needs the residuals
// clear of the subnormal range: sx >= 2^-100 with |h/sx| >= 1/4.  A smaller
// quotient may end an ulp off, but it rounds to the code 0 either way.
__device__ inline uint32_t corrected_code_bits(float h, float sx, float inv) {
    const float q0 = h * inv;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-sx, q0, h), inv, q0);
    const float q2 = __builtin_fmaf(__builtin_fmaf(-sx, q1, h), inv, q1);
    return __float_as_uint(q2 + kRoundMagic);
}
// bytes 0..3 <- low bytes of b0..b3
__device__ inline uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
    return __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u) | __builtin_amdgcn_perm(b3, b2, 0x04000C0Cu);
}

#pragma clang fp contract(on)

// bf16 bits of f, rounded to nearest even (finite inputs)
__device__ inline uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- cross-lane reductions (DPP within 16-lane rows, then the four rows) ----
template <int CTRL>
__device__ inline int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_HMIRROR = 0x141;  // lane i <-> 7 - i within 8 lanes
constexpr int DPP_MIRROR = 0x140;   // lane i <-> 15 - i within 16 lanes

// Max over the wave (wave-uniform result).
__device__ inline float wave_max(float v) {
    v = fmaxf(v, __int_as_float(dpp<DPP_XOR1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp<DPP_XOR2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp<DPP_HMIRROR>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp<DPP_MIRROR>(__float_as_int(v))));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

template <int CTRL>
__device__ inline double dpp_d(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = dpp<CTRL>((int)(b & 0xFFFFFFFFll));
    const int hi = dpp<CTRL>((int)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ inline double readlane_d(double v, int l) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), l);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
// Sum over the wave in one fixed tree order (wave-uniform result).
__device__ inline double wave_sum(double v) {
    v += dpp_d<DPP_XOR1>(v);
    v += dpp_d<DPP_XOR2>(v);
    v += dpp_d<DPP_HMIRROR>(v);
    v += dpp_d<DPP_MIRROR>(v);
    return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}

// Thread -> activation mapping.  Each thread holds up to NCH 16-byte chunks of
// its row's slice (a chunk is 4 fp32 or 8 bf16 elements): WPR waves per row,
// row m = wave / WPR, chunk c = it + i * TPR for i < NCH.  `nw` counts the
// iterations i in which the wave has at least one chunk, so a wave skips the
// rest with a uniform branch.
template <int XT, int EPT>
struct Act {
    static constexpr int E = XT == 0 ? 4 : 8;      // elements per chunk
    static constexpr int NCH = EPT / E;            // chunks per thread (EPT elements)
    static constexpr int ES = XT == 0 ? 4 : 2;     // bytes per element
    int m;      // row of this wave; >= M: the wave holds no activations
    int it;     // thread index within the row
    int tpr;    // threads per row
    int cpr;    // chunks per row of the slice
    int nw;     // wave-uniform
};

template <int XT, int EPT>
__device__ inline Act<XT, EPT> act_map(const KArgs& a, uint32_t wt, int lane) {
    Act<XT, EPT> am;
    am.m = (wt >> 10) & 15;
    am.it = ((wt >> 14) & 31) * 64 + lane;
    am.tpr = a.tpr;
    am.cpr = a.cpr;
    am.nw = (wt >> 19) & 15;
    return am;
}

// Chunk index of a thread's i-th chunk.  The wave-uniform part goes through
// readfirstlane so it stays a scalar added to the lane's index: folded into a
// 64-bit multiply-add instead, the unused high half of its addend can land on
// a register a load is still filling, and the wait for it would serialise the
// activation loads.
template <int XT, int EPT>
__device__ inline int chunk_of(const Act<XT, EPT>& am, int i) {
    return am.it + __builtin_amdgcn_readfirstlane(i * am.tpr);
}

// Raw 16-byte chunks of slice [k_lo, k_lo + KS) (SwiGLU: gate in xr, up in ur).
// The loads go through a buffer resource spanning the row's slice: a chunk past
// its end reads zeros, and the chunks of steps i >= nw are not loaded (zero),
// so every invalid element is 0 without a select.
template <int PRO, int XT, int EPT>
__device__ inline void load_act(const KArgs& a, const Act<XT, EPT>& am, int k_lo,
                                uint4 xr[Act<XT, EPT>::NCH], uint4 ur[Act<XT, EPT>::NCH]) {
    constexpr int CB = Act<XT, EPT>::E * Act<XT, EPT>::ES;     // 16 bytes per chunk
    // the row's slice start (wave-uniform) and this thread's byte offsets in it
    const int64_t row = ((int64_t)am.m * a.ld + k_lo) * Act<XT, EPT>::ES;
    const int nrec = am.cpr * CB;
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(a.x)) + row, (short)0, nrec, kRsrcFlags);
    __amdgpu_buffer_rsrc_t us = xs;
    if (PRO == PRO_SWIGLU)
        us = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(static_cast<const uint8_t*>(a.x2)) + row,
                                               (short)0, nrec, kRsrcFlags);
#pragma unroll
    for (int i = 0; i < Act<XT, EPT>::NCH; ++i) {
        xr[i] = make_uint4(0u, 0u, 0u, 0u);
        ur[i] = make_uint4(0u, 0u, 0u, 0u);
        if (i < am.nw) {
            const int off = chunk_of(am, i) * CB;
            xr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xs, off, 0, 0));
            if (PRO == PRO_SWIGLU)
                ur[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(us, off, 0, 0));
        }
    }
}

template <int XT, int EPT>
__device__ inline void load_gamma(const KArgs& a, const Act<XT, EPT>& am, int k_lo,
                                  float g[Act<XT, EPT>::NCH * Act<XT, EPT>::E]) {
    constexpr int E = Act<XT, EPT>::E;
#pragma unroll
    for (int i = 0; i < Act<XT, EPT>::NCH; ++i) {
#pragma unroll
        for (int e = 0; e < E; ++e) g[i * E + e] = 0.0f;
        if (i < am.nw) {
            const int c = chunk_of(am, i);
            const int cc = c < am.cpr ? c : 0;
            const float4* gp = reinterpret_cast<const float4*>(a.gamma + k_lo + (int64_t)cc * E);
#pragma unroll
            for (int v = 0; v < E / 4; ++v) {
                const float4 t = gp[v];
                g[i * E + 4 * v] = t.x; g[i * E + 4 * v + 1] = t.y;
                g[i * E + 4 * v + 2] = t.z; g[i * E + 4 * v + 3] = t.w;
            }
        }
    }
}

// h values of the thread's chunks (SwiGLU applied); invalid elements are 0.
template <int PRO, int XT, int EPT>
__device__ inline void finish_act(const Act<XT, EPT>& am, const uint4 xr[Act<XT, EPT>::NCH],
                                  const uint4 ur[Act<XT, EPT>::NCH], float h[Act<XT, EPT>::NCH * Act<XT, EPT>::E]) {
    constexpr int E = Act<XT, EPT>::E;
#pragma unroll
    for (int i = 0; i < Act<XT, EPT>::NCH; ++i) {
        const uint32_t xw[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
        const uint32_t uw[4] = {ur[i].x, ur[i].y, ur[i].z, ur[i].w};
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float xv, uv;
            if (XT == 0) {
                xv = __uint_as_float(xw[e]);
                uv = __uint_as_float(uw[e]);
            } else {
                xv = __uint_as_float((e & 1) ? (xw[e >> 1] & 0xFFFF0000u) : (xw[e >> 1] << 16));
                uv = __uint_as_float((e & 1) ? (uw[e >> 1] & 0xFFFF0000u) : (uw[e >> 1] << 16));
            }
            // invalid elements load as 0, and every prologue maps 0 to 0
            h[i * E + e] = (PRO == PRO_SWIGLU) ? silu_mul(xv, uv) : xv;
        }
    }
}

template <int XT, int EPT>
__device__ inline double sum_sq(const float h[Act<XT, EPT>::NCH * Act<XT, EPT>::E]) {
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < Act<XT, EPT>::NCH * Act<XT, EPT>::E; ++j) ss += (double)h[j] * (double)h[j];
    return ss;
}
// max |h| as an integer maximum of the magnitude bits (equal to the float
// maximum for finite values, and cheaper: no NaN handling).
template <int XT, int EPT>
__device__ inline float abs_max(const float h[Act<XT, EPT>::NCH * Act<XT, EPT>::E]) {
    uint32_t mx = 0u;
#pragma unroll
    for (int j = 0; j < Act<XT, EPT>::NCH * Act<XT, EPT>::E; ++j) mx = max(mx, __float_as_uint(h[j]) & 0x7FFFFFFFu);
    return __uint_as_float(mx);
}
// The same for bf16 activations taken as they are, on the packed words: a
// packed 16-bit maximum of the magnitude bits, two elements per operation.
template <int EPT>
__device__ inline float abs_max_bf16(const uint4 xr[Act<1, EPT>::NCH]) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 mx = {0, 0};
#pragma unroll
    for (int i = 0; i < Act<1, EPT>::NCH; ++i) {
        const uint32_t w[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, w[d] & 0x7FFF7FFFu));
    }
    const uint32_t top = max((uint32_t)mx.x, (uint32_t)mx.y);
    return __uint_as_float(top << 16);
}

// A row's slice statistic from its waves' values, in wave order.
// Sum over the waves of row m (m wave-uniform): lane k of each 16-lane row takes
// wave k's value (0 for the waves of other rows), then a fixed tree within the
// 16 lanes leaves the sum in every lane (each step adds two equal-shaped halves,
// so every lane computes the same sum, in the same order every launch).
__device__ inline double row_sum_d(const KArgs& a, const Smem& sm, int m) {
    const int k = threadIdx.x & 15;
    const int lo = m * a.WPR;
    const double w = sm.wd[k];
    double v = (k >= lo && k < lo + a.WPR) ? w : 0.0;
    v += dpp_d<DPP_XOR1>(v);
    v += dpp_d<DPP_XOR2>(v);
    v += dpp_d<DPP_HMIRROR>(v);
    v += dpp_d<DPP_MIRROR>(v);
    return v;
}
// A row's slice statistic from its waves' values in ascending wave order, as a
// short loop: these run once per launch from a cold instruction cache, where
// every 64 bytes of code cost about 0.1 us.
__device__ inline double combine_d(const KArgs& a, const Smem& sm, int m) {
    double v = 0.0;
#pragma nounroll
    for (int w = m * a.WPR; w < (m + 1) * a.WPR; ++w) v += sm.wd[w];
    return v;
}
__device__ inline float combine_f(const KArgs& a, const Smem& sm, int m) {
    float v = 0.0f;
#pragma nounroll
    for (int w = m * a.WPR; w < (m + 1) * a.WPR; ++w) v = fmaxf(v, sm.wf[w]);
    return v;
}
// Max over the waves of row m (m wave-uniform): lane k of each 16-lane row
// takes wave k's value, and a max within the row leaves the result in every
// lane.  Values are >= 0, so 0 stands in for waves of other rows.
__device__ inline float row_max(const KArgs& a, const Smem& sm, int m, int lane) {
    const int k = lane & 15;
    const int lo = m * a.WPR;
    const float w = sm.wf[k];
    float v = (k >= lo && k < lo + a.WPR) ? w : 0.0f;
    v = fmaxf(v, __int_as_float(dpp<DPP_XOR1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp<DPP_XOR2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp<DPP_HMIRROR>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp<DPP_MIRROR>(__float_as_int(v))));
    return v;
}
// Row m's statistic over all slices (S > 1), slices in ascending order.
__device__ inline double slices_sum(const KArgs& a, const Smem& sm, int m) {
    const double2* p = reinterpret_cast<const double2*>(sm.exd + m * SMAX);
    double s = 0.0;
    for (int q = 0; q < a.S; q += 2) {
        const double2 t = p[q >> 1];
        s += t.x;
        if (q + 1 < a.S) s += t.y;
    }
    return s;
}
__device__ inline float slices_max(const KArgs& a, const Smem& sm, int m) {
    const float4* p = reinterpret_cast<const float4*>(sm.exf + m * SMAX);
    float s = 0.0f;
    for (int q = 0; q < a.S; q += 4) {
        const float4 t = p[q >> 2];
        s = fmaxf(s, t.x);
        if (q + 1 < a.S) s = fmaxf(s, t.y);
        if (q + 2 < a.S) s = fmaxf(s, t.z);
        if (q + 3 < a.S) s = fmaxf(s, t.w);
    }
    return s;
}

// Statistics of slice `sl`, computed locally when its exchange word did not
// arrive in time.  Same thread mapping and summation order as the workgroups
// that own that slice, so the result is bit-identical.  All threads call it.
template <int PRO, int XT, int EPT>
__device__ inline void slice_stat(const KArgs& a, Smem& sm, uint32_t wt, int lane, int wv, int sl,
                                  bool want_ss) {
    constexpr int E = Act<XT, EPT>::E;
    const Act<XT, EPT> am = act_map<XT, EPT>(a, wt, lane);
    uint4 xr[Act<XT, EPT>::NCH], ur[Act<XT, EPT>::NCH];
    float h[Act<XT, EPT>::NCH * E];
    load_act<PRO, XT, EPT>(a, am, sl * a.KS, xr, ur);
    finish_act<PRO, XT, EPT>(am, xr, ur, h);
    if (want_ss) {
        const double ss = wave_sum(sum_sq<XT, EPT>(h));
        if (lane == 0) sm.wd[wv] = ss;
    } else {
        if (PRO == PRO_RMSNORM) {
            float g[Act<XT, EPT>::NCH * E];
            load_gamma<XT, EPT>(a, am, sl * a.KS, g);
            const float r = (am.m < a.m) ? sm.rr[am.m] : 1.0f;
#pragma unroll
            for (int j = 0; j < Act<XT, EPT>::NCH * E; ++j) h[j] = rms_apply(h[j], r, g[j]);
        }
        const float mx = wave_max(abs_max<XT, EPT>(h));
        if (lane == 0) sm.wf[wv] = mx;
    }
    __syncthreads();
    if (threadIdx.x < a.m) {
        if (want_ss) sm.exd[threadIdx.x * SMAX + sl] = combine_d(a, sm, threadIdx.x);
        else sm.exf[threadIdx.x * SMAX + sl] = combine_f(a, sm, threadIdx.x);
    }
    __syncthreads();
}

// How long the chiplet-local exchange words are polled before the
// device-scope ones, in ticks of the 100 MHz constant clock.
#ifndef SK_XCD_POLL_TICKS
#define SK_XCD_POLL_TICKS 200
#endif
constexpr uint64_t kXcdPollTicks = SK_XCD_POLL_TICKS;

// Exchange of this slice's per-row value with the other slices (S > 1), run by
// the poller wave only, after the waves' values are in sm.wd / sm.wf.  Every
// word carries the call's tag in its high half, so no fence is needed: a
// reader simply waits until all words show the tag.  absmax: one word
// (tag | float bits).  Sum of squares (double): two words (tag | high half),
// (tag | low half).  Word j = sl * 8 + row of slice sl.
//
// The code is kept short on purpose: one wave runs it once per launch from a
// cold instruction cache, where every 64 bytes of code cost about 0.1 us.
//
// absmax with the slices on one XCD: the slices of a range are workgroups r,
// r + R, r + 2R, ...; with R a multiple of the 8 chiplets and round-robin
// dispatch they share an XCD, so a word stored through the L1 into that XCD's
// L2 (sc0) is seen there by the other slices' polls within a few hundred ns.
// The device-scope copy is written only after this wave's polls: its write is
// acknowledged once it has gone out to memory, and every poll's wait would
// wait for that acknowledgement too (a wave's vector memory operations
// complete in order).  A poll that sees nothing on the chiplet for
// kXcdPollTicks (the slices sit on other XCDs) turns to the device-scope copy.
__device__ inline void exchange_publish(const KArgs& a, Smem& sm, int lane, int s, bool is_ss) {
    if (lane >= a.m) return;
    const u64 tag = (u64)sm.tag << 32;
    const int j = s * 8 + lane;
    if (is_ss) {
        const double v = combine_d(a, sm, lane);
        sm.exd[lane * SMAX + s] = v;
        const u64 bits = (u64)__double_as_longlong(v);
        __hip_atomic_store(&a.ws->ssh[j], tag | (bits >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.ws->ssl[j], tag | (bits & 0xFFFFFFFFull), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        const float v = combine_f(a, sm, lane);
        sm.exf[lane * SMAX + s] = v;
        const u64 w = tag | __float_as_uint(v);
        if ((a.R & 7) == 0)
            __asm__ volatile("global_store_dwordx2 %0, %1, off sc0" ::"v"(&a.ws->amax_xcd[j]), "v"(w) : "memory");
        else
            __hip_atomic_store(&a.ws->amax[j], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ inline void exchange_poll(const KArgs& a, Smem& sm, int lane, int s, bool is_ss) {
    const uint32_t tag = sm.tag;
    const bool xcd = !is_ss && (a.R & 7) == 0;
    if (lane < SMAX) sm.miss[lane] = 0;
#pragma nounroll
    for (int j = lane; j < a.S * 8; j += 64) {
        const int sl = j >> 3, mm = j & 7;
        if (sl == s || mm >= a.m) continue;
        const u64* p = is_ss ? &a.ws->ssh[j] : xcd ? &a.ws->amax_xcd[j] : &a.ws->amax[j];
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        bool ok = false;
#pragma nounroll
        for (int it = 0; it < a.spin_limit; ++it) {
            const u64 v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t lo = (uint32_t)v;
            bool seen = (uint32_t)(v >> 32) == tag;
            if (is_ss) {
                const u64 w = __hip_atomic_load(&a.ws->ssl[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                seen = seen && (uint32_t)(w >> 32) == tag;
                if (seen) sm.exd[mm * SMAX + sl] = __longlong_as_double((long long)(((u64)lo << 32) | (uint32_t)w));
            } else if (seen) {
                sm.exf[mm * SMAX + sl] = __uint_as_float(lo);
            }
            if (seen) {
                ok = true;
                break;
            }
            if (__builtin_amdgcn_s_memrealtime() - t0 > kXcdPollTicks) p = is_ss ? p : &a.ws->amax[j];
            __builtin_amdgcn_s_sleep(1);
        }
        if (!ok) sm.miss[sl] = 1;          // every writer stores the same value
    }
    if (xcd && lane < a.m)
        __hip_atomic_store(&a.ws->amax[s * 8 + lane], ((u64)tag << 32) | __float_as_uint(sm.exf[lane * SMAX + s]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// y of output row omm in tile ot from its scaled sum: sx * sum, or NaN for a
// tile of an expert-bank call whose listed id lies outside the bank.
// Entry i of the expert list (i wave-uniform), by a scalar load: the list is
// read-only during the launch, and a vector load's wait would also wait for
// every activation and weight load the wave has in flight.
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ inline int expert_id(const KArgs& a, int i) {
    return ((const_i32*)(a.experts))[__builtin_amdgcn_readfirstlane(i)];
}

// Index in the expert list of logical tile t (t < 2^20), without a division.
__device__ inline int tile_expert(const KArgs& a, int t) {
    return (int)(((u64)(uint32_t)t * a.tpe_magic) >> 40);
}

__device__ inline float out_value(const KArgs& a, const Smem& sm, int ot, int omm, float sum) {
    if (a.tpe) {
        const int e = expert_id(a, tile_expert(a, ot));
        if (e < 0 || e >= a.n_experts) return __builtin_nanf("");
    }
    return sm.sx[omm] * sum;
}

// --------------------------------------------------------------------------
// the kernel
// --------------------------------------------------------------------------

template <int FMT, int PRO, int XT, int GS, bool DOT4, bool DBG, bool CANON, bool WIDE, int PD>
__global__ __launch_bounds__(NT) void gemm_kernel(KArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ Smem sm;
    constexpr bool CB = FMT == FMT_CB;          // codebook levels instead of integer weights
    constexpr int NG = (GS == 0) ? 8 : 4 / GS;  // groups per super-block (GS = 0: G = 16)
    // G = 32 on the v_dot4 path: one 4-byte scale load per lane per slot instead
    // of the row's four (16 bytes, the same for the four lanes of a column); the
    // lanes trade block sums instead (see the v_dot4 step of `process`)
    constexpr bool SCALE1 = SK_SCALE1 && NG == 4 && DOT4 && !CB;
    constexpr bool REST_IN_Q = SK_REST_IN_Q && !CB && (SK_REST_IN_Q > 1 || !DOT4);
    // The weight bytes fed to the dot products hold w scaled by 16 (W4: the
    // nibble in the byte's top half) or 4 (W6: the 6 bits in the top of the
    // byte), so sign extension is free; the sums are scaled back at the store.
    constexpr int WSH = (FMT == FMT_W6) ? 2 : 4;
    constexpr float KINV = CB ? 1.0f : (FMT == FMT_W6) ? 0.25f : 0.0625f;
    // Activations per thread: 16 on v_dot4 or with a prologue, 32 on the MFMA
    // path without one.  The wide instances (used only where they save
    // K-slices: their larger prologue code costs the other calls time) take 24
    // on v_dot4 (K = 17408 in one slice), and 40 on the MFMA path without a
    // prologue or with the RMSNorm prologue for a single K-slice and 4-bit
    // weights: compiling out the cross-slice exchange (ONE), and keeping gamma
    // in LDS rather than beside each activation, is what makes room for the
    // latter (the 6-bit unpack needs a few registers more than are left).
    constexpr bool ONE = WIDE && PRO == PRO_RMSNORM && !DOT4;
    constexpr int EPT = DOT4 ? (WIDE ? 24 : 16) : (PRO == PRO_NONE || ONE) ? (WIDE ? 40 : 32) : 16;
    constexpr int E = Act<XT, EPT>::E;
    constexpr int NCH = Act<XT, EPT>::NCH;
    constexpr int PIPE = PD ? PD : pipe_of(DOT4, CB);   // PD: a depth other than the path's own
    constexpr int PRIME = DOT4 ? kPrimeDot4 : kPrimeMfma;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    // The entry block of the arguments, all requested before anything waits on
    // one of them (otherwise the first loads would wait for a chain of
    // dependent argument fetches).
    __asm__ volatile("" ::"s"(a.data), "s"(a.x), "s"(a.ld), "s"(a.tile_full), "s"(a.rag_w), "s"(a.rag_s),
                     "s"(a.m), "s"(a.KS), "s"(a.S), "s"(a.KBs), "s"(a.tq), "s"(a.trem), "s"(a.jn0),
                     "s"(a.jn1), "s"(a.TW), "s"(a.spw), "s"(a.srem), "s"(a.KB), "s"(a.sbf), "s"(a.swo), "s"(a.t_rag),
                     "s"(a.nr_last), "s"(a.rag_sbw), "s"(a.rag_sbs), "s"(a.cpr), "s"(a.tpr), "s"(a.tpe),
                     "s"(a.wtab[wv]));
    const int nl = lane & 15;
    const int hl = lane >> 4;
    const int M = DOT4 ? 1 : a.m;                 // the v_dot4 instances run M = 1 only
    const int r = blockIdx.x;
    const int s = blockIdx.y;
    const int k_lo = s * a.KS;

    // 1. the activations first: they head the longest dependency chain (x ->
    //    statistics -> q -> every dot product), so their loads go out before
    //    any other address arithmetic; then the call's tag and the weight stream
    //    (a wave's loads complete in issue order)
    const uint32_t wt = a.wtab[wv];
    const Act<XT, EPT> am = act_map<XT, EPT>(a, wt, lane);
    uint4 xr[NCH], ur[NCH];
    // RMSNorm: the slice's gamma, float4 i = tid + j * NT, on its way to LDS.  A
    // slice holds at most EPT activations per thread of its row, and a row has
    // all NT threads only at M = 1 (v_dot4, or the codebook), NT / 2 or fewer
    // otherwise: EPT / 4, or EPT / 8, float4 per thread (and K <= 17408).
    constexpr int GQ_ROWS = (DOT4 || CB) ? EPT / 4 : EPT / 8;
    constexpr int GQ_MAXK = (int)((kMaxGemmK / 4 + NT - 1) / NT);
    constexpr int GQ = (PRO != PRO_RMSNORM) ? 1 : GQ_ROWS < GQ_MAXK ? GQ_ROWS : GQ_MAXK;
    float4 gq[GQ];
    // Split path (PRO_QIN): the slice's q arrives ready, M rows of KS / 8
    // octets; thread tid takes octets tid + i * NT, QMAX per pass.
    constexpr int QMAX = 4;
    const int q_oct = a.KS / 8;
    const int q_total = M * q_oct;
    uint2 qr[QMAX];
    auto q_load = [&](const int pass) {
#pragma unroll
        for (int i = 0; i < QMAX; ++i) {
            const int o = (pass * QMAX + i) * NT + tid;
            const int mq = o / q_oct, ko = o - mq * q_oct;
            qr[i] = (o < q_total) ? *reinterpret_cast<const uint2*>(
                        static_cast<const int8_t*>(a.x) + (int64_t)mq * a.k + k_lo + ko * 8)
                                  : make_uint2(0u, 0u);
        }
    };
    if constexpr (PRO == PRO_QIN) {
        q_load(0);
    } else {
        load_act<PRO, XT, EPT>(a, am, k_lo, xr, ur);
        if (PRO == PRO_RMSNORM) {
            // every row scales by the same gamma: it is loaded once per
            // workgroup, coalesced, and kept in LDS instead of in registers
            // beside each activation
            const float4* gp = reinterpret_cast<const float4*>(a.gamma + k_lo);
#pragma unroll
            for (int j = 0; j < GQ; ++j)
                gq[j] = ((tid + j * NT) * 4 < a.KS) ? gp[tid + j * NT] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }

    // The launch generation (K-split launches only), after the activation
    // loads: it is a device-scope round trip, and loads complete in issue
    // order, so the activations must not queue behind it.  (The compiler waits
    // for it right away; the K-split launches run on the MFMA path, which waits
    // for its activations before the weight stream anyway.)
    uint32_t gen = 0;
    if (!ONE && a.S > 1) gen = __hip_atomic_load(&a.ws->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // work assignment: block (r, s) owns tiles [t_begin, t_end) of K-slice s;
    // wave wv works on tile group tg (every TW-th tile) and super-blocks
    // [kw * spw, (kw + 1) * spw) of the slice
    const int kb_lo = s * a.KBs;
    const bool big = r < a.trem;
    const int t_begin = r * a.tq + (big ? r : a.trem);
    const int t_end = t_begin + a.tq + (big ? 1 : 0);
    const int jn = big ? a.jn1 : a.jn0;         // tiles per group, padded
    const int tg = wt & 31;
    const int kw = (wt >> 5) & 31;
    // the wave's k-part of the slice: spw super-blocks, one more for the first
    // srem k-parts (K-split launches, where the slice's count has few divisors)
    const int spw_w = a.spw + (kw < a.srem ? 1 : 0);
    const int kwo = kw * a.spw + min(kw, a.srem);   // its first super-block in the slice
    const int kbw = kb_lo + kwo;
    // With S > 1 the last wave only runs the cross-slice exchange: it never has
    // weight loads in flight, so its polls are not queued behind them.
    const bool poller = !ONE && (a.S > 1) && (wv == NW - 1);
    const bool active = tg < a.TW && !poller;

    // LDS: [q: M x ks int8][sums of q][wave partials, two halves]
    // (codebook: [16 levels as bf16 hi|lo pairs][q as bf16: M x ks bytes][wave partials])
    uint32_t* lut_l = reinterpret_cast<uint32_t*>(lds);
    int8_t* q_l = reinterpret_cast<int8_t*>(lds + (CB ? 64 : 0));
    float* red_l = reinterpret_cast<float*>(q_l + (size_t)M * a.ks);
    float* gam_l = red_l + 2 * a.red_half;        // RMSNorm: the slice's gamma, KS floats
    float* fix_l = gam_l + (PRO == PRO_RMSNORM ? a.KS : 0);   // chunks to redo, kFixCap entries
    constexpr bool FIXLIST = !DBG && !CB && PRO != PRO_QIN;
    // the partials' padding entries must read as zero: clear both halves (the
    // first tile step's barrier orders this before any partial is written)
    for (int i = tid; i < a.red_half / 2; i += NT)
        reinterpret_cast<float4*>(red_l)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);

    // Slots: the wave's weight stream is a sequence of super-blocks, spw per
    // tile step, walked in groups of PIPE slots (a tile step's last group is
    // padded when PIPE does not divide spw); tile step j is tile
    // t_begin + tg + j * TW.  Tile steps [0, jw) hold work; every wave walks jn
    // of them (the tile barriers).  Padding slots and the steps past jw load
    // in-bounds stand-in bytes and skip the arithmetic.
    const int ntile = t_end - t_begin;
    // tiles tg, tg + TW, ... below ntile: jn = ceil(ntile / TW) of them, one
    // fewer for the groups past the last step's share
    const int jw = active ? jn - (tg >= ntile - (jn - 1) * a.TW ? 1 : 0) : 0;
    const int ngrp = (spw_w + PIPE - 1) / PIPE;      // slot groups per tile step

    // Per-lane byte offsets inside a super-block: a full tile (16 rows) and the
    // weight's ragged last tile (nr_last rows; its lanes nl >= nr_last read
    // offset 0 and feed only their own, never stored, row).  Offsets of a full
    // tile stay inside the weight's first super-block, so a stand-in slot can
    // read them from base 0.
    const int nr_rag = a.nr_last;
    const bool lane_rag_ok = nl < nr_rag;
    const int lw_full = lane * 16, lw_rag = lane_rag_ok ? (hl * nr_rag + nl) * 16 : 0;
    const int lh_full = 16 * 64 + lane * 8, lh_rag = lane_rag_ok ? nr_rag * 64 + (hl * nr_rag + nl) * 8 : 0;
    const int ls_full = nl * NG * 4, ls_rag = lane_rag_ok ? nl * NG * 4 : 0;

    // Load-side cursor: group lg of tile step lj.  Its slots' weights start at
    // byte offset gw of the weight and step by gws; their scales sit gso bytes
    // after the weights and step by gss; grg marks the ragged tile; gnv counts
    // the slots that hold work.  All of it is wave-uniform and set once per
    // group, so a slot's load is a few scalar operations.  The loads go through
    // a buffer resource based at the group's first byte: padding slots and
    // stand-in groups (no work) use an offset past the resource, which reads
    // zeros without a memory access, so every wave issues the same loads (the
    // compiler's wait counts stay exact) and no stand-in load costs bandwidth.
    int lj = 0, lg = 0;
    int64_t gw = 0;
    int gso = 0, gws = 0, gss = 0, gnv = 0;
    bool grg = false;
    __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.data), (short)0, 0, kRsrcFlags);
    // canonical layout (CANON, W4 only): per-lane offsets of the group's tile
    // (rows past N read row N - 1; those lanes' sums are never stored)
    int64_t gs = 0;
    int glw = 0, gls = 0;
    const int rb = a.k / 2;                          // bytes per canonical weight row
    auto group_setup = [&]() {
        const int t = t_begin + tg + lj * a.TW;
        const bool valid = lj < jw;
        const int kb = kbw + lg * PIPE;
        gnv = valid ? min(PIPE, spw_w - lg * PIPE) : 0;
        if constexpr (CANON) {
            const int tt = valid ? t : 0;
            const int nlc = min(tt * TILE_ROWS + nl, a.n - 1) - tt * TILE_ROWS;
            glw = nlc * rb + 4 * hl;
            gls = nlc * a.kg * 4;
            gw = !valid ? 0 : (int64_t)tt * TILE_ROWS * rb + (int64_t)kb * 64;
            gs = (int64_t)a.n * rb + (!valid ? 0 : ((int64_t)tt * TILE_ROWS * a.kg + (int64_t)kb * NG) * 4);
            gws = !valid ? 0 : 64;
            gss = !valid ? 0 : NG * 4;
        } else {
            grg = valid && t == a.t_rag;
            // the bank's tile behind logical tile t (expert banks), else t; a
            // stand-in group maps tile 0 so the list is never read past its end,
            // and an id outside the bank reads expert 0 (its rows are written as NaN)
            const int tv = valid ? t : 0;
            int tb = t;
            if (a.tpe) {
                const int li = tile_expert(a, tv);
                const int e = expert_id(a, li);
                tb = ((e >= 0 && e < a.n_experts) ? e : 0) * a.tpe + (tv - li * a.tpe);
            }
            const int64_t wo = (int64_t)tb * a.tile_full + (int64_t)kb * a.sbf;
            gw = !valid ? 0 : grg ? a.rag_w + (int64_t)kb * a.rag_sbw : wo;
            // scales relative to the weights: the ragged tile keeps them after all
            // of its weight parts, (KB - kb) weight parts and kb scale parts on
            gso = grg ? (a.KB - kb) * a.rag_sbw + kb * a.rag_sbs : a.swo;
            gws = grg ? a.rag_sbw : a.sbf;
            gss = grg ? a.rag_sbs : a.sbf;
            grs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.data) + gw, (short)0,
                                                    valid ? kRsrcMax : 0, kRsrcFlags);
        }
    };
    auto group_next = [&]() {
        if (++lg == ngrp) {
            lg = 0;
            ++lj;
        }
        group_setup();
    };
    group_setup();
    // Slot d of the load group into registers.  Every wave issues the same
    // load instructions, so the compiler's wait counts are exact.
    auto load_slot = [&](const int d, uint4& w4, uint2& h2, float4& sv, float4& sv2) {
        if constexpr (CANON) {
            // octet hl of each 32-k block j: 4 bytes, 16 bytes apart in the row
            // (padding slots re-read slot 0)
            const int dd = d < gnv ? d : 0;
            const uint32_t* p = reinterpret_cast<const uint32_t*>(a.data + gw + dd * gws + glw);
            w4 = make_uint4(__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 4),
                            __builtin_nontemporal_load(p + 8), __builtin_nontemporal_load(p + 12));
            const float* sp = reinterpret_cast<const float*>(a.data + gs + dd * gss + gls);
            if (NG == 8) {
                sv = make_float4(__builtin_nontemporal_load(sp), __builtin_nontemporal_load(sp + 1),
                                 __builtin_nontemporal_load(sp + 2), __builtin_nontemporal_load(sp + 3));
                sv2 = make_float4(__builtin_nontemporal_load(sp + 4), __builtin_nontemporal_load(sp + 5),
                                  __builtin_nontemporal_load(sp + 6), __builtin_nontemporal_load(sp + 7));
            } else if (NG == 4 && SCALE1) {
                sv = make_float4(__builtin_nontemporal_load(sp + hl), 0.0f, 0.0f, 0.0f);
            } else if (NG == 4) {
                sv = make_float4(__builtin_nontemporal_load(sp), __builtin_nontemporal_load(sp + 1),
                                 __builtin_nontemporal_load(sp + 2), __builtin_nontemporal_load(sp + 3));
            } else if (NG == 2) {
                sv = make_float4(__builtin_nontemporal_load(sp), __builtin_nontemporal_load(sp + 1), 0.0f, 0.0f);
            } else {
                sv = make_float4(__builtin_nontemporal_load(sp), 0.0f, 0.0f, 0.0f);
            }
        } else {
            const bool on = d < gnv;
            const int lw = grg ? lw_rag : lw_full;
            const int ls = grg ? ls_rag : ls_full;
            const int wo = on ? d * gws + lw : kOutside;
            const int so = on ? gso + d * gss + ls : kOutside;
            w4 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(grs, wo, 0, kStreamPolicy));
            if (FMT == FMT_W6)
                h2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                   grs, on ? d * gws + (grg ? lh_rag : lh_full) : kOutside, 0,
                                                   kStreamPolicy));
            if (NG == 8) {
                sv = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(grs, so, 0, kStreamPolicy));
                sv2 = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(grs, on ? so + 16 : kOutside, 0,
                                                                                       kStreamPolicy));
            } else if (NG == 4 && SCALE1) {
                // one scale per lane, s[row nl][block hl]
                sv = make_float4(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                               grs, on ? so + 4 * hl : kOutside, 0, kStreamPolicy)),
                                 0.0f, 0.0f, 0.0f);
            } else if (NG == 4) {
                sv = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(grs, so, 0, kStreamPolicy));
            } else if (NG == 2) {
                const float2 v = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(grs, so, 0, kStreamPolicy));
                sv = make_float4(v.x, v.y, 0.0f, 0.0f);
            } else {
                sv = make_float4(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(grs, so, 0, kStreamPolicy)),
                                 0.0f, 0.0f, 0.0f);
            }
        }
    };

    // M >= 2 (more activation loads, and with S > 1 every slice's statistics
    // gate the exchange): a wave's weight stream starts once its own
    // activations are in, so they do not queue behind a burst of cold weight
    // requests.  Waiting for the whole workgroup's (a barrier) was slower: the
    // waves whose activations arrive first then sit idle.
    if (!DOT4 && SK_MFMA_ACT_FIRST) {
        __builtin_amdgcn_s_waitcnt(0xF70);    // vmcnt(0)
        if (SK_MFMA_ACT_FIRST == 1) __syncthreads();
    }
    uint4 wbuf[PIPE];
    uint2 hbuf[PIPE];
    float4 sbuf[PIPE], sbuf2[PIPE];
#pragma unroll
    for (int d = 0; d < PRIME; ++d) load_slot(d, wbuf[d], hbuf[d], sbuf[d], sbuf2[d]);
    bool rest_done = false;

    // 2. activation prologue: per-row statistics of h, then q into LDS
    if (!ONE && a.S > 1 && tid == 0) sm.tag = gen + 1u;
    if (CB && tid < 16) {
        // each level as a bf16 pair hi + lo (|level - hi - lo| <= 2^-17 |level|)
        const float v = a.codebook[tid];
        const uint32_t hi = bf16_rne(v);
        const uint32_t lo = bf16_rne(v - __uint_as_float(hi << 16));
        lut_l[tid] = hi | (lo << 16);
    }
    if constexpr (PRO == PRO_QIN) {
        // the ready-made q octets into LDS (same order as the quantiser's), then sx
        for (int pass = 0; pass * QMAX * NT < q_total; ++pass) {
            if (pass > 0) q_load(pass);
#pragma unroll
            for (int i = 0; i < QMAX; ++i) {
                const int o = (pass * QMAX + i) * NT + tid;
                if (o < q_total) {
                    const int mq = o / q_oct, ko = o - mq * q_oct;
                    const int ow = ko & 15;
                    const int pos = (ko >> 4) * 128 + ((ow & 3) * 4 + (ow >> 2)) * 8;
                    *reinterpret_cast<uint2*>(q_l + mq * a.ks + pos) = qr[i];
                }
            }
        }
        if (tid < M) sm.sx[tid] = static_cast<const float*>(a.x2)[tid];
    } else {
        // bf16 activations taken as they are: their maximum from the packed
        // words, before they are widened (the raw words are dead after that)
        float mx_packed = 0.0f;
        if constexpr (PRO == PRO_NONE && XT == 1) mx_packed = abs_max_bf16<EPT>(xr);
        float h[NCH * E];
        finish_act<PRO, XT, EPT>(am, xr, ur, h);
        const int mrow = am.m < M ? am.m : 0;
        const bool row_lead = lane == 0 && am.m < M && am.it == 0;   // one thread per row

        if (PRO == PRO_RMSNORM) {
            const double ss = wave_sum(sum_sq<XT, EPT>(h));
            if (lane == 0) sm.wd[wv] = ss;
#pragma unroll
            for (int j = 0; j < GQ; ++j)
                if ((tid + j * NT) * 4 < a.KS) reinterpret_cast<float4*>(gam_l)[tid + j * NT] = gq[j];
            __syncthreads();
            double tot;
            if (ONE || a.S == 1) {
                tot = row_sum_d(a, sm, mrow);
            } else {
                if (poller) {
                    exchange_publish(a, sm, lane, s, true);
                    exchange_poll(a, sm, lane, s, true);
                }
                __syncthreads();
                for (int sl = 0; sl < a.S; ++sl)
                    if (sm.miss[sl]) slice_stat<PRO, XT, EPT>(a, sm, wt, lane, wv, sl, true);
                tot = slices_sum(a, sm, mrow);
            }
            const float ms = (float)(tot / (double)a.k);
            const float d = ms + a.eps;
            const float sd = (float)__builtin_sqrt((double)d);   // correctly rounded fp32 sqrt
            const float rr = (float)(1.0 / (double)sd);          // correctly rounded fp32 1/x
            if (row_lead) sm.rr[am.m] = rr;
            // chunk i of this thread is elements c E .. c E + E - 1 of the slice;
            // a chunk past the row (h = 0 there) reads the row's last gamma
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int cc = min(chunk_of(am, i), am.cpr - 1);
                const float4* gp = reinterpret_cast<const float4*>(gam_l + cc * E);
#pragma unroll
                for (int v = 0; v < E / 4; ++v) {
                    const float4 g4 = gp[v];
                    const int j = i * E + 4 * v;
                    h[j] = rms_apply(h[j], rr, g4.x);
                    h[j + 1] = rms_apply(h[j + 1], rr, g4.y);
                    h[j + 2] = rms_apply(h[j + 2], rr, g4.z);
                    h[j + 3] = rms_apply(h[j + 3], rr, g4.w);
                }
            }
        }
        float amx;
        {
            const float mx = wave_max((PRO == PRO_NONE && XT == 1) ? mx_packed : abs_max<XT, EPT>(h));
            if (lane == 0) sm.wf[wv] = mx;
            __syncthreads();
            if (ONE || a.S == 1) {
                amx = row_max(a, sm, mrow, lane);
            } else {
                if (poller) {
                    exchange_publish(a, sm, lane, s, false);
                    exchange_poll(a, sm, lane, s, false);
                }
                __syncthreads();
                for (int sl = 0; sl < a.S; ++sl)
                    if (sm.miss[sl]) slice_stat<PRO, XT, EPT>(a, sm, wt, lane, wv, sl, false);
                amx = slices_max(a, sm, mrow);
            }
        }
        const float sx = (amx > 0.0f) ? amx / 127.0f : 0.0f;
        const float inv = (sx > 0.0f) ? 1.0f / sx : 0.0f;   // sx == 0: every code is 0
        if (row_lead) {
            sm.sx[am.m] = sx;
            if (DBG && a.sx_out && r == 0 && s == 0) a.sx_out[am.m] = sx;
        }

        // quantise this slice into LDS (straight-line code: it runs once per
        // launch, so every instruction of it is a cold instruction-cache fetch)
        // LDS order of q: in each 128-k super-block, octet 4j + h is stored at
        // position 4h + j, so a lane's four octets are contiguous.  Chunk i of a
        // thread is TPR chunks (a multiple of 128 elements) after chunk 0, so its
        // position is chunk 0's plus i whole super-blocks.
        const int c0 = am.it;
        const int o0 = (c0 * E) >> 3, ow0 = o0 & 15;
        const int pos0 = (o0 >> 4) * 128 + ((ow0 & 3) * 4 + (ow0 >> 2)) * 8 + ((c0 * E) & 7);
        const int pstep = am.tpr * E;
        if (FIXLIST && am.nw > 0) {
            // One chunk at a time: its codes from the bracketing products, then
            // (if an element's products round apart) a place in the wave's list
            // of chunks to redo, then its store, so only one chunk's codes are
            // live at a time.  A wave holds one activation row, so sx and the
            // tiny-scale branch are wave-uniform.
            const float inv_lo = inv * kInvLo, inv_hi = inv * kInvHi;
            const bool tiny = sx < kMinCorrectedSx && sx > 0.0f;
            int nfix_w = 0;                                       // chunks this wave listed
            float* const fix_w = fix_l + wv * (kWaveFix * kFixStride);
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                uint32_t bc[E];
                uint32_t split = 0;
#pragma unroll
                for (int e = 0; e < E; ++e) bc[e] = code_bits(h[i * E + e], inv_lo, inv_hi, split);
                if (__builtin_expect(tiny, 0)) {
#pragma unroll
                    for (int e = 0; e < E; ++e) bc[e] = __float_as_uint(h[i * E + e] / sx + kRoundMagic);
                } else {
                    const bool redo = split != 0;
                    const uint64_t bal = __ballot(redo);
                    if (bal) {
                        const int idx = nfix_w + (int)__builtin_amdgcn_mbcnt_hi(
                                                     (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                        if (redo) {
                            if (idx < kWaveFix) {
                                float4* en = reinterpret_cast<float4*>(fix_w + idx * kFixStride);
                                en[0] = make_float4(h[i * E], h[i * E + 1], h[i * E + 2], h[i * E + 3]);
                                if (E == 8) en[1] = make_float4(h[i * E + 4 % E], h[i * E + 5 % E], h[i * E + 6 % E],
                                                                h[i * E + 7 % E]);
                                fix_w[idx * kFixStride + 8] = __int_as_float(pos0 + i * pstep);
                            } else {
#pragma unroll
                                for (int e = 0; e < E; ++e) bc[e] = corrected_code_bits(h[i * E + e], sx, inv);
                            }
                        }
                        nfix_w += (int)__builtin_popcountll(bal);
                    }
                }
                int8_t* dst = q_l + am.m * a.ks + pos0 + i * pstep;
                if (i < am.nw && chunk_of(am, i) < am.cpr) {
                    if (E == 4) *reinterpret_cast<uint32_t*>(dst) = pack_low_bytes(bc[0], bc[1], bc[2], bc[3]);
                    else *reinterpret_cast<uint2*>(dst) = make_uint2(pack_low_bytes(bc[0], bc[1], bc[2], bc[3]),
                                                                     pack_low_bytes(bc[4 % E], bc[5 % E], bc[6 % E],
                                                                                    bc[7 % E]));
                }
                // one more slot of the first group after each chunk but the last:
                // the address unit is idle while the quantiser runs, and a burst
                // of loads here would hold the waves at issue
                if (REST_IN_Q && PRIME + i < PIPE && i + 1 < NCH)
                    load_slot(PRIME + i, wbuf[PRIME + i], hbuf[PRIME + i], sbuf[PRIME + i], sbuf2[PRIME + i]);
            }
            if (REST_IN_Q) {
#pragma unroll
                for (int d = PRIME + NCH - 1; d < PIPE; ++d) load_slot(d, wbuf[d], hbuf[d], sbuf[d], sbuf2[d]);
                rest_done = true;
            }
            if (nfix_w > 0) {
                // the listed chunks, element by element over the wave's lanes,
                // written over the codes stored above (a wave's LDS operations
                // complete in order)
                const int nel = min(nfix_w, kWaveFix) * E;
                for (int t = lane; t < nel; t += 64) {
                    const float* en = fix_w + (t / E) * kFixStride;
                    const uint32_t cbits = corrected_code_bits(en[t % E], sx, inv);
                    q_l[am.m * a.ks + __float_as_int(en[8]) + t % E] = (int8_t)cbits;
                }
            }
        } else if (am.nw > 0) {
            // Codes of all elements from the bracketing products, noting the chunks
            // that hold an element whose products round apart.  Such elements are
            // common (with bf16 data most rows have some), so their chunks are
            // redone with the corrected quotient: a few short blocks, each skipped
            // by the waves that do not need it, rather than a division per
            // element, whose cold code would cost more than the quantiser.
            uint32_t b[NCH * E];
            uint32_t rare = 0;             // bit i: chunk i needs the corrected quotient
            const float inv_lo = inv * kInvLo, inv_hi = inv * kInvHi;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                uint32_t split = 0;
#pragma unroll
                for (int e = 0; e < E; ++e) b[i * E + e] = code_bits(h[i * E + e], inv_lo, inv_hi, split);
                rare |= (split != 0 ? 1u : 0u) << i;
            }
            if (__builtin_expect(sx < kMinCorrectedSx && sx > 0.0f, 0)) {
#pragma unroll
                for (int j = 0; j < NCH * E; ++j) b[j] = __float_as_uint(h[j] / sx + kRoundMagic);
            } else if (__builtin_expect(rare != 0, 0)) {
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    if (rare & (1u << i)) {
#pragma unroll
                        for (int e = 0; e < E; ++e) b[i * E + e] = corrected_code_bits(h[i * E + e], sx, inv);
                    }
                }
            }
            uint32_t pk[NCH * E / 4];
#pragma unroll
            for (int w = 0; w < NCH * E / 4; ++w) pk[w] = pack_low_bytes(b[4 * w], b[4 * w + 1], b[4 * w + 2], b[4 * w + 3]);
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const uint32_t* pc = pk + i * (E / 4);
                const bool ok = i < am.nw && chunk_of(am, i) < am.cpr;
                const int pos = pos0 + i * pstep;
                if (CB) {
                    // bf16 copies of q (exact: |q| <= 127), two per dword
                    uint32_t hb[E / 2];
#pragma unroll
                    for (int e2 = 0; e2 < E / 2; ++e2) {
                        const int q0 = (int)(int8_t)(pc[(2 * e2) / 4] >> (8 * ((2 * e2) % 4)));
                        const int q1 = (int)(int8_t)(pc[(2 * e2 + 1) / 4] >> (8 * ((2 * e2 + 1) % 4)));
                        hb[e2] = (__float_as_uint((float)q0) >> 16) | (__float_as_uint((float)q1) & 0xFFFF0000u);
                    }
                    uint8_t* dst = reinterpret_cast<uint8_t*>(q_l) + am.m * a.ks + pos * 2;
                    if (ok) {
                        if (E == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(hb[0], hb[1]);
                        else *reinterpret_cast<uint4*>(dst) = make_uint4(hb[0], hb[1], hb[2], hb[E / 2 - 1]);
                    }
                } else {
                    int8_t* dst = q_l + am.m * a.ks + pos;
                    if (ok) {
                        if (E == 4) *reinterpret_cast<uint32_t*>(dst) = pc[0];
                        else *reinterpret_cast<uint2*>(dst) = make_uint2(pc[0], pc[E / 4 - 1]);
                    }
                }
            }
            if (DBG && a.q_out && r == 0) {          // debug export of q
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    const int c = chunk_of(am, i);
                    if (i < am.nw && c < am.cpr) {
                        int8_t* gq = a.q_out + (int64_t)am.m * a.k + k_lo + c * E;
                        if (E == 4) *reinterpret_cast<uint32_t*>(gq) = pk[i];
                        else *reinterpret_cast<uint2*>(gq) = make_uint2(pk[2 * i], pk[2 * i + 1]);
                    }
                }
            }
        }
    }
    // The rest of the first group's loads (unless the quantiser issued them) and
    // the next group's cursor go out before the workgroup waits for q: waves
    // without activations get there first and, with the loop set-up after them,
    // bring that code into the instruction cache (empty at every launch) while
    // the others quantise.
    // On the v_dot4 path a wave whose whole share is one load group and that
    // quantised issues that group's rest after the barrier instead: those loads
    // queue behind the other waves' (issued right after the statistics), and
    // the barrier would wait for the queue.  With more groups the wave's stream
    // is long and the late start costs more than the barrier saves.
    const bool late_rest = DOT4 && am.nw > 0 && !rest_done && jn * ngrp == 1;
    if (!rest_done && !late_rest) {
#pragma unroll
        for (int d = PRIME; d < PIPE; ++d) load_slot(d, wbuf[d], hbuf[d], sbuf[d], sbuf2[d]);
    }
    if (!late_rest) group_next();

    // 3. stream the weights: a register pipeline of PIPE slots in flight
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // A-operand row (activation row) of this lane.  Rows past M repeat row
    // M - 1: their products land in output rows >= M, which are never stored,
    // so the LDS reads need no mask.
    const int ml = nl < M ? nl : M - 1;
    // consume slot (weights w_in/h_in, scales s_in) of tile t whose super-block
    // is kbr within the slice; `work` is false for padding and stand-in slots
    auto process = [&](const bool work, const int t, const int kbr, const uint4 w_in, const uint2 h_in,
                       const float4 s_in, const float4 s_in2) {
        // Every slot's registers count as read here, valid or not, so the
        // compiler waits for exactly this slot's loads (a skipped read would
        // leave them pending when the next load reuses the registers).
        if (FMT == FMT_W6) __asm__ volatile("" ::"v"(w_in.x), "v"(h_in.x), "v"(s_in.x));
        else if (CANON) __asm__ volatile("" ::"v"(w_in.x), "v"(w_in.y), "v"(w_in.z), "v"(w_in.w), "v"(s_in.x));
        else __asm__ volatile("" ::"v"(w_in.x), "v"(s_in.x));
        if (work) {
            const int kb = kb_lo + kbr;
            // Lanes of rows past the weight's end (ragged last tile) hold
            // stand-in bytes; they only ever feed their own row's sums, which are
            // never stored.
            const bool row_ok = t != a.t_rag || lane_rag_ok;
            const uint32_t wd[4] = {w_in.x, w_in.y, w_in.z, w_in.w};
            const float sv[4] = {s_in.x, s_in.y, s_in.z, s_in.w};
            // lo[j] / hi[j]: the bytes of codes e = 0..3 / 4..7 of octet hl of block j,
            // each as a signed byte equal to w << WSH
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (FMT == FMT_W6) {
                    const uint32_t hd = (j < 2) ? h_in.x : h_in.y;
                    const uint32_t hlo = (j & 1) ? (hd << 2) : (hd << 6);   // bits 4-5 of code c
                    const uint32_t hhi = (j & 1) ? hd : (hd << 4);          // bits 4-5 of code c + 4
                    lo[j] = ((wd[j] << 2) & 0x3C3C3C3Cu) | (hlo & 0xC0C0C0C0u);
                    hi[j] = ((wd[j] >> 2) & 0x3C3C3C3Cu) | (hhi & 0xC0C0C0C0u);
                } else if (CANON) {
                    // canonical bytes hold codes (2i, 2i + 1) in (low, high) nibbles
                    const uint32_t ev = (wd[j] << 4) & 0xF0F0F0F0u;   // codes 0, 2, 4, 6
                    const uint32_t od = wd[j] & 0xF0F0F0F0u;          // codes 1, 3, 5, 7
                    lo[j] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
                    hi[j] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
                } else {
                    lo[j] = (wd[j] << 4) & 0xF0F0F0F0u;
                    hi[j] = wd[j] & 0xF0F0F0F0u;
                }
            }
            const int kbase = kbr * 128;          // slice-relative k of this super-block
            // q of this lane: octet hl of each 32-k block j, stored contiguously
            const uint4* qp = reinterpret_cast<const uint4*>(q_l + (DOT4 ? 0 : ml * a.ks) + kbase + hl * 32);
            if (CB) {
                // Codebook: each level is hi + lo in bf16, so the per-group sum of
                // level * q is two bf16 MFMAs with fp32 accumulation (products exact).
                // A = q as bf16 (row ml, octet hl of block j); B = the levels of this
                // lane's 8 codes, built from the 16-entry table in LDS.
                const uint4* qbp = reinterpret_cast<const uint4*>(
                    reinterpret_cast<const uint8_t*>(q_l) + ml * a.ks + (kbase + hl * 32) * 2);
                const float sv8[8] = {s_in.x, s_in.y, s_in.z, s_in.w, s_in2.x, s_in2.y, s_in2.z, s_in2.w};
                v4f cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 qa = qbp[j];
                    uint32_t ent[8];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        ent[c] = lut_l[(wd[j] >> (8 * c)) & 15u];          // element c
                        ent[c + 4] = lut_l[(wd[j] >> (8 * c + 4)) & 15u];  // element c + 4
                    }
                    uint4 bh, bl;                 // elements (0,1) (2,3) (4,5) (6,7)
                    bh.x = __builtin_amdgcn_perm(ent[1], ent[0], 0x05040100u);
                    bh.y = __builtin_amdgcn_perm(ent[3], ent[2], 0x05040100u);
                    bh.z = __builtin_amdgcn_perm(ent[5], ent[4], 0x05040100u);
                    bh.w = __builtin_amdgcn_perm(ent[7], ent[6], 0x05040100u);
                    bl.x = __builtin_amdgcn_perm(ent[1], ent[0], 0x07060302u);
                    bl.y = __builtin_amdgcn_perm(ent[3], ent[2], 0x07060302u);
                    bl.z = __builtin_amdgcn_perm(ent[5], ent[4], 0x07060302u);
                    bl.w = __builtin_amdgcn_perm(ent[7], ent[6], 0x07060302u);
                    const bf16x8 B_hi = __builtin_bit_cast(bf16x8, bh);
                    const bf16x8 B_lo = __builtin_bit_cast(bf16x8, bl);
                    if (NG == 8) {
                        // G = 16: octets 0-1 of the block are group 2j, octets 2-3 group 2j+1
                        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
                        const bf16x8 A_e = __builtin_bit_cast(bf16x8, hl < 2 ? qa : z);
                        const bf16x8 A_o = __builtin_bit_cast(bf16x8, hl < 2 ? z : qa);
                        v4f ce = {0.0f, 0.0f, 0.0f, 0.0f}, co = ce;
                        ce = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_e, B_hi, ce, 0, 0, 0);
                        ce = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_e, B_lo, ce, 0, 0, 0);
                        co = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_o, B_hi, co, 0, 0, 0);
                        co = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_o, B_lo, co, 0, 0, 0);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            acc[rr] = __builtin_fmaf(sv8[2 * j], ce[rr], acc[rr]);
                            acc[rr] = __builtin_fmaf(sv8[2 * j + 1], co[rr], acc[rr]);
                        }
                    } else {
                        const bf16x8 A = __builtin_bit_cast(bf16x8, qa);
                        cg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B_hi, cg, 0, 0, 0);
                        cg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B_lo, cg, 0, 0, 0);
                        if ((j + 1) % (GS ? GS : 1) == 0) {
#pragma unroll
                            for (int rr = 0; rr < 4; ++rr) acc[rr] = __builtin_fmaf(sv[j / (GS ? GS : 1)], cg[rr], acc[rr]);
                            cg = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                        }
                    }
                }
            } else if (DOT4) {
                const uint4 q01 = qp[0], q23 = qp[1];
                const uint32_t qw[8] = {q01.x, q01.y, q01.z, q01.w, q23.x, q23.y, q23.z, q23.w};
                int part[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = __builtin_amdgcn_sdot4((int)hi[j], (int)qw[2 * j + 1], 0, false);
                    part[j] = __builtin_amdgcn_sdot4((int)lo[j], (int)qw[2 * j], c, false);
                }
                int pg[NG];
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    pg[gi] = 0;
#pragma unroll
                    for (int jj = 0; jj < GS; ++jj) pg[gi] += part[gi * GS + jj];
                }
                if (SCALE1) {
                    // Transpose-reduce over the four 16-lane rows (lane swaps
                    // move whole rows, so every lane keeps its column nl): lane
                    // (nl, hl) ends with the sum of block hl's four octets for
                    // row nl and needs one scale, s[nl][hl], the one it loaded.
                    // Rows 0-1 and 2-3 trade blocks 2-3 for 0-1 and add; then
                    // odd and even rows trade and add.
                    const auto x02 = __builtin_amdgcn_permlane32_swap((uint32_t)pg[0], (uint32_t)pg[2], false, false);
                    const auto x13 = __builtin_amdgcn_permlane32_swap((uint32_t)pg[1], (uint32_t)pg[3], false, false);
                    const auto y = __builtin_amdgcn_permlane16_swap(x02[0] + x02[1], x13[0] + x13[1], false, false);
                    acc[0] = __builtin_fmaf(sv[0], (float)(int)(y[0] + y[1]), acc[0]);
                } else {
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi) acc[0] = __builtin_fmaf(sv[gi], (float)pg[gi], acc[0]);
                }
                if (DBG && a.p_out) {        // debug export: this lane's share of each group partial
                    if (row_ok) {
#pragma unroll
                        for (int gi = 0; gi < NG; ++gi)
                            atomicAdd(&a.p_out[((int64_t)t * TILE_ROWS + nl) * a.kg + kb * NG + gi],
                                      pg[gi] >> WSH);
                    }
                }
            } else {
                const uint4 q01 = qp[0], q23 = qp[1];
                const long av[4] = {(long)((uint64_t)q01.x | ((uint64_t)q01.y << 32)),
                                    (long)((uint64_t)q01.z | ((uint64_t)q01.w << 32)),
                                    (long)((uint64_t)q23.x | ((uint64_t)q23.y << 32)),
                                    (long)((uint64_t)q23.z | ((uint64_t)q23.w << 32))};
                long bv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) bv[j] = (long)((uint64_t)lo[j] | ((uint64_t)hi[j] << 32));
                // every group's MFMAs first (independent, so they issue back to
                // back), then the scaling
                v4i c[NG];
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    c[gi] = v4i{0, 0, 0, 0};
#pragma unroll
                    for (int jj = 0; jj < GS; ++jj)
                        c[gi] = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[gi * GS + jj],
                                                                     bv[gi * GS + jj], c[gi], 0, 0, 0);
                }
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) acc[rr] = __builtin_fmaf(sv[gi], (float)c[gi][rr], acc[rr]);
                    if (DBG && a.p_out) {    // debug export of the group partials
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int mm = 4 * hl + rr;
                            if (mm < M && row_ok)
                                a.p_out[((int64_t)mm * a.n + (int64_t)t * TILE_ROWS + nl) * a.kg +
                                        kb * NG + gi] = c[gi][rr] >> WSH;
                        }
                    }
                }
            }
        }
    };

    // 4. tile epilogue of tile step j with this lane's sums v4: fixed-order sum
    //    of the waves' partials.  The partials buffer alternates between two
    //    halves, so one barrier per tile is enough (a wave cannot reuse a half
    //    before every thread passed the next barrier).
    // The partials are stored output-major, [row][column][wave] with a pitch of
    // kRedPitch floats, so one thread reads all the waves' values of its output
    // with four 16-byte LDS reads (the 16 lanes of a row write to distinct banks).
    auto tile_epilogue = [&](const float* v4, const int j) {
        float* red = red_l + (j & 1) * a.red_half;
        if (DOT4) {
            // the four k-quarters of a row sit 16 lanes apart
            float v = v4[0];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            if (active && lane < 16) red[(tg * 16 + nl) * a.kwp + kw] = v;
        } else if (active) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int mm = 4 * hl + rr;
                if (mm < M) red[((tg * M + mm) * 16 + nl) * a.kwp + kw] = v4[rr];
            }
        }
        __syncthreads();
        const int nout = a.TW * M * 16;
        if (tid < nout) {
            // output (tile group ogrp, row omm, column onn) of thread tid:
            // tid / 16 = ogrp * M + omm, divided by M through a multiply
            const int o16 = tid >> 4;
            const int ogrp = DOT4 ? o16 : (o16 * a.m_magic) >> 16;
            const int omm = DOT4 ? 0 : o16 - ogrp * M;
            const int onn = tid & 15;
            const int ot = t_begin + ogrp + j * a.TW;
            if (ot < t_end) {
                // the KW k-parts of tile group ogrp, added in k order (then the
                // zero padding); all reads go out first: one LDS round trip
                const float4* rp = reinterpret_cast<const float4*>(red + (o16 * 16 + onn) * a.kwp);
                float4 t4[4];
                t4[0] = rp[0];
                t4[1] = t4[2] = t4[3] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (a.kwp > 4) t4[1] = rp[1];
                if (a.kwp > 8) {
                    t4[2] = rp[2];
                    t4[3] = rp[3];
                }
                float osum = 0.0f;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    osum += t4[q4].x;
                    osum += t4[q4].y;
                    osum += t4[q4].z;
                    osum += t4[q4].w;
                }
                if (ONE || a.S == 1) {
                    if (ot * TILE_ROWS + onn < a.n)
                        a.y[(int64_t)omm * a.n + (int64_t)ot * TILE_ROWS + onn] = out_value(a, sm, ot, omm, osum * KINV);
                } else {
                    const u64 v = ((u64)sm.tag << 32) | __float_as_uint(osum);
                    __hip_atomic_store(&a.part[(((int64_t)ot * a.S + s) * M + omm) * 16 + onn], v,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    };

    for (int pj = 0; pj < jn; ++pj) {
        if (pj == 0) {
            __syncthreads();                    // q (and sx) complete in LDS
            if (late_rest) {
#pragma unroll
                for (int d = PRIME; d < PIPE; ++d) load_slot(d, wbuf[d], hbuf[d], sbuf[d], sbuf2[d]);
                group_next();
            }
        }
        const bool pvalid = pj < jw;
        const int t = t_begin + tg + pj * a.TW;
        for (int pg = 0; pg < ngrp; ++pg) {
            const int pnv = pvalid ? min(PIPE, spw_w - pg * PIPE) : 0;
            const int kb0 = kwo + pg * PIPE;
#pragma unroll
            for (int d = 0; d < PIPE; ++d) {
                process(d < pnv, t, kb0 + d, wbuf[d], hbuf[d], sbuf[d], sbuf2[d]);
                load_slot(d, wbuf[d], hbuf[d], sbuf[d], sbuf2[d]);
            }
            group_next();
        }
        tile_epilogue(acc, pj);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[rr] = 0.0f;
    }

    // 5. merge the slices' partials: the last of range r's S workgroups to
    //    arrive adds them, for every tile of the range, in slice order
    if (!ONE && a.S > 1) {
        __syncthreads();
        // counted by the poller wave (the last one): it stored no partials,
        // so the count's round trip does not wait behind their writes
        if (tid == (NW - 1) * 64) {
            const uint32_t old = __hip_atomic_fetch_add(&a.ws->cnt[r], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int lst = old == (uint32_t)(a.S - 1);
            if (lst) __hip_atomic_store(&a.ws->cnt[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sm.last = lst;
        }
        __syncthreads();
        if (sm.last) {
            // The partials' first reads go out together and through this XCD's
            // L2 (sc0: past the CU's L1), where the slices of the range wrote
            // them when they share the XCD; a word whose tag is not there yet
            // (or that sits in another XCD's L2) is then read at device scope.
            const __amdgpu_buffer_rsrc_t prs =
                __builtin_amdgcn_make_buffer_rsrc(a.part, (short)0, kRsrcMax, kRsrcFlags);
            constexpr int kSc0 = 1;
            for (int e = tid; e < ntile * M * 16; e += NT) {
                const int ci = e / (M * 16);
                const int omm = (e / 16) % M;
                const int onn = e & 15;
                const int ot = t_begin + ci;
                float tot = 0.0f;
                for (int sl0 = 0; sl0 < a.S; sl0 += 4) {
                    u64 v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int sl = min(sl0 + u, a.S - 1);
                        const int off = (int)(((((int64_t)ot * a.S + sl) * M + omm) * 16 + onn) * 8);
                        v[u] = __builtin_bit_cast(u64, __builtin_amdgcn_raw_buffer_load_b64(prs, off, 0, kSc0));
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int sl = sl0 + u;
                        if (sl >= a.S) break;
                        // Every partial was stored before its workgroup counted itself, so
                        // its tag shows up shortly; the bound only guards against a hang (a
                        // missing partial would turn y into NaN rather than stall the GPU).
                        const u64* p = &a.part[(((int64_t)ot * a.S + sl) * M + omm) * 16 + onn];
                        u64 w = v[u];
                        for (int it = 0; (uint32_t)(w >> 32) != sm.tag && it < (1 << 24); ++it)
                            w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        tot += ((uint32_t)(w >> 32) == sm.tag) ? __uint_as_float((uint32_t)w) : __builtin_nanf("");
                    }
                }
                if (ot * TILE_ROWS + onn < a.n)
                    a.y[(int64_t)omm * a.n + (int64_t)ot * TILE_ROWS + onn] = out_value(a, sm, ot, omm, tot * KINV);
            }
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

// Kernel pointer for a format, prologue, activation dtype, groups per 32-k block
// (gs; 0 = the codebook's G = 16), M = 1 / M >= 2 and the wide activation budget
// (M >= 2: no prologue with W4 or W6, RMSNorm with W4); nullptr if not built.
template <int FMT, int PRO, int XT, int GS, bool DBG>
KernelFn pick_dot(bool dot4, bool wide) {
    if constexpr (FMT == FMT_CB) {
        return gemm_kernel<FMT, PRO, XT, GS, false, DBG, false, false, 0>;   // the codebook runs on MFMA for every M
    } else if constexpr (PRO == PRO_NONE) {
        if (dot4)
            return wide ? gemm_kernel<FMT, PRO, XT, GS, true, DBG, false, true, 0>
                        : gemm_kernel<FMT, PRO, XT, GS, true, DBG, false, false, 0>;
        return wide ? gemm_kernel<FMT, PRO, XT, GS, false, DBG, false, true, 0>
                    : gemm_kernel<FMT, PRO, XT, GS, false, DBG, false, false, 0>;
    } else if constexpr (PRO == PRO_RMSNORM && FMT == FMT_W4) {
        return dot4 ? gemm_kernel<FMT, PRO, XT, GS, true, DBG, false, false, 0>
               : wide ? gemm_kernel<FMT, PRO, XT, GS, false, DBG, false, true, 0>
                      : gemm_kernel<FMT, PRO, XT, GS, false, DBG, false, false, 0>;
    } else {
        return dot4 ? gemm_kernel<FMT, PRO, XT, GS, true, DBG, false, false, 0>
                    : gemm_kernel<FMT, PRO, XT, GS, false, DBG, false, false, 0>;
    }
}
template <int FMT, int PRO, int XT, bool DBG>
KernelFn pick_gs(int gs, bool dot4, bool wide) {
    switch (gs) {
        case 0:
            if constexpr (FMT == FMT_CB) return pick_dot<FMT, PRO, XT, 0, DBG>(dot4, wide);
            return nullptr;
        case 1: return pick_dot<FMT, PRO, XT, 1, DBG>(dot4, wide);
        case 2: return pick_dot<FMT, PRO, XT, 2, DBG>(dot4, wide);
        default: return pick_dot<FMT, PRO, XT, 4, DBG>(dot4, wide);
    }
}
template <int FMT, int PRO, bool DBG>
KernelFn pick_xt(int xt, int gs, bool dot4, bool wide) {
    return xt == 1 ? pick_gs<FMT, PRO, 1, DBG>(gs, dot4, wide) : pick_gs<FMT, PRO, 0, DBG>(gs, dot4, wide);
}
// 4-bit weights without a prologue and a pipeline of PD slots (the planner's
// choice where PD divides a wave's super-blocks per tile and the default does not)
template <int PD, int XT, int GS>
KernelFn pick_pipe_dot(bool dot4, bool wide) {
    if (dot4)
        return wide ? gemm_kernel<FMT_W4, PRO_NONE, XT, GS, true, false, false, true, PD>
                    : gemm_kernel<FMT_W4, PRO_NONE, XT, GS, true, false, false, false, PD>;
    return wide ? gemm_kernel<FMT_W4, PRO_NONE, XT, GS, false, false, false, true, PD>
                : gemm_kernel<FMT_W4, PRO_NONE, XT, GS, false, false, false, false, PD>;
}
template <int PD>
KernelFn pick_pipe(int xt, int gs, bool dot4, bool wide) {
    switch (gs * 2 + (xt == 1 ? 1 : 0)) {
        case 2: return pick_pipe_dot<PD, 0, 1>(dot4, wide);
        case 3: return pick_pipe_dot<PD, 1, 1>(dot4, wide);
        case 4: return pick_pipe_dot<PD, 0, 2>(dot4, wide);
        case 5: return pick_pipe_dot<PD, 1, 2>(dot4, wide);
        case 8: return pick_pipe_dot<PD, 0, 4>(dot4, wide);
        case 9: return pick_pipe_dot<PD, 1, 4>(dot4, wide);
        default: return nullptr;
    }
}
// The split path's kernels: 4-bit weights in the canonical layout, either
// quantising x in the launch (PRO_NONE) or reading q from memory (PRO_QIN,
// which has no activation budget).
template <int PRO, int XT, int GS>
KernelFn pick_canon_dot(bool dot4, bool wide) {
    if constexpr (PRO == PRO_NONE) {
        if (!dot4 && wide) return gemm_kernel<FMT_W4, PRO, XT, GS, false, false, true, true, 0>;
        if (dot4 && wide) return gemm_kernel<FMT_W4, PRO, XT, GS, true, false, true, true, 0>;
    }
    return dot4 ? gemm_kernel<FMT_W4, PRO, XT, GS, true, false, true, false, 0>
                : gemm_kernel<FMT_W4, PRO, XT, GS, false, false, true, false, 0>;
}
template <int PRO, int XT>
KernelFn pick_canon_gs(int gs, bool dot4, bool wide) {
    switch (gs) {
        case 1: return pick_canon_dot<PRO, XT, 1>(dot4, wide);
        case 2: return pick_canon_dot<PRO, XT, 2>(dot4, wide);
        case 4: return pick_canon_dot<PRO, XT, 4>(dot4, wide);
        default: return nullptr;
    }
}

template <int FMT, bool DBG>
KernelFn pick_format(int pro, int xt, int gs, bool dot4, bool wide) {
    switch (pro) {
        case PRO_RMSNORM: return pick_xt<FMT, PRO_RMSNORM, DBG>(xt, gs, dot4, wide);
        case PRO_SWIGLU: return pick_xt<FMT, PRO_SWIGLU, DBG>(xt, gs, dot4, false);
        default: return pick_xt<FMT, PRO_NONE, DBG>(xt, gs, dot4, wide);
    }
}

}  // namespace

}  // namespace sk

#endif  // SK_GEMM_KERNEL_H
