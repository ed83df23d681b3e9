// sk_api.hip -- the C ABI: host-side validation, then dispatch to the kernels.
//
// Every check runs on the host before any HIP call, so a rejected call has
// touched neither the device nor the caller's memory.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "../../include/sk_repack.h"
#include "../../include/sk_repack_test.h"
#include "sk_internal.h"

#define SK_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using sk::Geom;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int format_bits(int fmt) { return fmt == SK_W6_SYM ? 6 : 4; }

// The page's shape rules for the format ("Comfy quantization formats", format options).
bool page_shape_ok(int fmt, int64_t k, int64_t g) {
    if (g <= 0 || k <= 0 || k % g != 0) return false;
    if (fmt == SK_W6_SYM) return k % 32 == 0 && g % 16 == 0;
    return k % 16 == 0 && g >= 4 && (16 % g == 0 || g % 16 == 0);
}

bool backend_group_ok(int fmt, int64_t g) {
    if (fmt == SK_W4_CODEBOOK) return g == 16 || g == 32 || g == 64 || g == 128;
    return g == 32 || g == 64 || g == 128;
}

// Checks shared by every entry point that takes a weight.
sk_status check_weight(const sk_weight* w) {
    if (!w || !w->data) return SK_ERR_NULL;
    if (w->format != SK_W4_SYM && w->format != SK_W4_CODEBOOK && w->format != SK_W6_SYM)
        return SK_ERR_FORMAT;
    if (w->reserved != 0) return SK_ERR_FORMAT;
    if ((w->format == SK_W4_CODEBOOK) != (w->codebook != nullptr)) return SK_ERR_FORMAT;
    if (w->n < 1 || w->k < 1) return SK_ERR_SHAPE;
    if (!page_shape_ok(w->format, w->k, w->group)) return SK_ERR_SHAPE;
    const int64_t n = w->n, k = w->k, g = w->group;
    const size_t want = (size_t)(n * k * format_bits(w->format) / 8 + n * (k / g) * 4);
    if (w->bytes != want) return SK_ERR_SHAPE;
    if (!aligned16(w->data) || (w->codebook && !aligned16(w->codebook))) return SK_ERR_ALIGN;
    if (w->layout != SK_LAYOUT_CANONICAL && w->layout != SK_LAYOUT_STREAM) return SK_ERR_LAYOUT;
    if (k % sk::SB_K != 0 || k > sk::kMaxGemmK || !backend_group_ok(w->format, g) ||
        n > (1 << 24))
        return SK_ERR_UNSUPPORTED;
    if (!sk::reorder_fits(sk::make_geom(n, k, g, w->format))) return SK_ERR_UNSUPPORTED;
    return SK_OK;
}

sk_status from_hip(hipError_t e) { return e == hipSuccess ? SK_OK : SK_ERR_HIP; }

int g_spin_limit = 0;   // test hook: exchange polls before the local fallback (0 = default)

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Checks for the GEMM entry points, then the launch.
sk_status run_gemm(const sk_weight* w, bool w6_entry, int prologue, const void* x, const void* x2,
                   int64_t ld, int xt, const float* gamma, float eps, int m, float* y,
                   int8_t* q_out, float* sx_out, int32_t* p_out, void* ws, size_t ws_bytes,
                   void* stream, bool any_format, bool canon = false, int rows_per_expert = 0,
                   const int32_t* experts = nullptr, int n_list = 0, bool validate_only = false) {
    sk_status s = check_weight(w);
    if (s != SK_OK) return s;
    if (canon && w->format != SK_W4_SYM) return SK_ERR_FORMAT;
    if (prologue == sk::PRO_QIN && !x2) return SK_ERR_NULL;
    if (!x || !y || (prologue == sk::PRO_SWIGLU && !x2) || (prologue == sk::PRO_RMSNORM && !gamma))
        return SK_ERR_NULL;
    if (xt != SK_F32 && xt != SK_BF16) return SK_ERR_FORMAT;
    if (!any_format) {
        if (w6_entry && w->format != SK_W6_SYM) return SK_ERR_FORMAT;
        if (!w6_entry && w->format == SK_W6_SYM) return SK_ERR_FORMAT;
    }
    if (p_out && w->format == SK_W4_CODEBOOK) return SK_ERR_FORMAT;
    if (m < 1 || m > 8) return SK_ERR_SHAPE;
    const int esize = (xt == SK_BF16) ? 2 : 4;
    if (prologue == sk::PRO_SWIGLU) {
        if (ld < w->k) return SK_ERR_SHAPE;
        if ((ld * esize) % 16 != 0) return SK_ERR_ALIGN;
    } else {
        ld = w->k;
    }
    if (!aligned16(x) || !aligned16(y) || (x2 && prologue != sk::PRO_QIN && !aligned16(x2)) ||
        (gamma && !aligned16(gamma)) ||
        (q_out && !aligned16(q_out)) || (p_out && !aligned16(p_out)))
        return SK_ERR_ALIGN;
    if (w->layout != (canon ? SK_LAYOUT_CANONICAL : SK_LAYOUT_STREAM)) return SK_ERR_LAYOUT;
    // expert bank: the call's output rows are n_list experts of rows_per_expert rows
    int64_t n_call = w->n;
    if (rows_per_expert) n_call = (int64_t)n_list * rows_per_expert;
    const Geom G = sk::make_geom(n_call, w->k, w->group, w->format);
    const sk::Plan plan = sk::gemm_plan(G, m, prologue);
    if (!plan.ok) return SK_ERR_UNSUPPORTED;
    const size_t need = sk::workspace_bytes(plan);
    if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return SK_ERR_WORKSPACE;
    if (validate_only) return SK_OK;

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p_out) {
        hipError_t e = hipMemsetAsync(p_out, 0, (size_t)m * w->n * (w->k / w->group) * 4, st);
        if (e != hipSuccess) return SK_ERR_HIP;
    }
    sk::GemmCall c;
    c.data = static_cast<const uint8_t*>(w->data);
    c.codebook = w->codebook;
    c.x = x;
    c.x2 = x2;
    c.ld = ld;
    c.xt = xt;
    c.gamma = gamma;
    c.eps = eps;
    c.prologue = prologue;
    c.m = m;
    c.y = y;
    c.q_out = q_out;
    c.sx_out = sx_out;
    c.p_out = p_out;
    c.spin_limit = g_spin_limit;
    c.canon = canon;
    c.rows_per_expert = rows_per_expert;
    c.n_list = n_list;
    c.n_experts = rows_per_expert ? w->n / rows_per_expert : 0;
    c.experts = experts;
    c.ws = need > 0 ? ws : nullptr;
    return from_hip(sk::launch_gemm(G, c, st));
}

}  // namespace

SK_EXPORT const char* sk_status_string(sk_status s) {
    // Callers may pass any integer (C enums are ints); read it as one, since
    // an out-of-range value loaded as the enum type is undefined in C++.
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
        case SK_OK: return "ok";
        case SK_ERR_NULL: return "a required pointer is NULL";
        case SK_ERR_SHAPE: return "shape rule violated (format rules, M range, bytes or ld)";
        case SK_ERR_ALIGN: return "pointer or row stride not 16-byte aligned";
        case SK_ERR_FORMAT: return "wrong format, dtype or codebook for this entry point";
        case SK_ERR_LAYOUT: return "weight is in the wrong layout for this call";
        case SK_ERR_HIP: return "HIP runtime error";
        case SK_ERR_UNSUPPORTED: return "shape not supported by this backend";
        case SK_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    }
    return "unknown status";
}

SK_EXPORT sk_status sk_repack_w4a8(sk_weight* w, void* stream) {
    sk_status s = check_weight(w);
    if (s != SK_OK) return s;
    if (w->layout != SK_LAYOUT_CANONICAL) return SK_ERR_LAYOUT;
    const Geom G = sk::make_geom(w->n, w->k, w->group, w->format);
    s = from_hip(sk::repack_device(static_cast<uint8_t*>(w->data), G, false,
                                   static_cast<hipStream_t>(stream)));
    if (s == SK_OK) w->layout = SK_LAYOUT_STREAM;
    return s;
}

SK_EXPORT sk_status sk_unrepack_w4a8(sk_weight* w, void* stream) {
    sk_status s = check_weight(w);
    if (s != SK_OK) return s;
    if (w->layout != SK_LAYOUT_STREAM) return SK_ERR_LAYOUT;
    const Geom G = sk::make_geom(w->n, w->k, w->group, w->format);
    s = from_hip(sk::repack_device(static_cast<uint8_t*>(w->data), G, true,
                                   static_cast<hipStream_t>(stream)));
    if (s == SK_OK) w->layout = SK_LAYOUT_CANONICAL;
    return s;
}

SK_EXPORT sk_status sk_gemm_workspace_size(int n, int k, int group, int format, int m, int prologue,
                                           size_t* bytes) {
    if (!bytes) return SK_ERR_NULL;
    if (format != SK_W4_SYM && format != SK_W4_CODEBOOK && format != SK_W6_SYM) return SK_ERR_FORMAT;
    if (prologue < sk::PRO_NONE || prologue > sk::PRO_SWIGLU) return SK_ERR_FORMAT;
    if (n < 1 || k < 1 || m < 1 || m > 8 || !page_shape_ok(format, k, group)) return SK_ERR_SHAPE;
    if (k % sk::SB_K != 0 || k > sk::kMaxGemmK || !backend_group_ok(format, group) || n > (1 << 24))
        return SK_ERR_UNSUPPORTED;
    const sk::Plan p = sk::gemm_plan(sk::make_geom(n, k, group, format), m, prologue);
    if (!p.ok) return SK_ERR_UNSUPPORTED;
    *bytes = sk::workspace_bytes(p);
    return SK_OK;
}

SK_EXPORT sk_status sk_gemm_w4a8(const sk_weight* w, const void* x, int xt, int m, float* y,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    return run_gemm(w, false, sk::PRO_NONE, x, nullptr, 0, xt, nullptr, 0.0f, m, y, nullptr,
                    nullptr, nullptr, workspace, workspace_bytes, stream, false);
}

namespace {

// Fixed device scratch of sk_gemm_w4a8_noalloc: one array per device (each GPU
// the library runs on holds its own copy until the process ends), used as the
// workspace of launches that split K.  Host code uses the per-device address
// from hipGetSymbolAddress, never the array's name.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ void clear_scratch_kernel(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

// The current device's scratch address; the first call on a device looks it
// up and enqueues a clear of the whole array on `st` (a kernel, so it may be
// captured: a captured clear runs before every replay, which is harmless).
hipError_t noalloc_scratch(hipStream_t st, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL(clear_scratch_kernel, dim3(256), dim3(256), 0, st, static_cast<uint4*>(p),
                           kNoAllocScratchBytes / 16);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

SK_EXPORT sk_status sk_gemm_w4a8_noalloc(const sk_weight* w, const void* x, int xt, int m, float* y,
                                         void* stream) {
    // the same checks as sk_gemm_w4a8 (validation never touches the device),
    // with the scratch's size standing in for the workspace's: a call that
    // would need more is SK_ERR_WORKSPACE
    const sk_status s = run_gemm(w, false, sk::PRO_NONE, x, nullptr, 0, xt, nullptr, 0.0f, m, y, nullptr,
                                 nullptr, nullptr, reinterpret_cast<void*>(static_cast<uintptr_t>(256)),
                                 kNoAllocScratchBytes, stream, false, false, 0, nullptr, 0,
                                 /*validate_only=*/true);
    if (s != SK_OK) return s;
    void* ws = nullptr;
    if (from_hip(noalloc_scratch(static_cast<hipStream_t>(stream), &ws)) != SK_OK) return SK_ERR_HIP;
    return run_gemm(w, false, sk::PRO_NONE, x, nullptr, 0, xt, nullptr, 0.0f, m, y, nullptr, nullptr,
                    nullptr, ws, kNoAllocScratchBytes, stream, false);
}

SK_EXPORT sk_status sk_gemm_w6a8(const sk_weight* w, const void* x, int xt, int m, float* y,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    return run_gemm(w, true, sk::PRO_NONE, x, nullptr, 0, xt, nullptr, 0.0f, m, y, nullptr,
                    nullptr, nullptr, workspace, workspace_bytes, stream, false);
}

SK_EXPORT sk_status sk_gemm_fused_rmsnorm(const sk_weight* w, const void* x, int xt,
                                          const float* gamma, float eps, int m, float* y,
                                          void* workspace, size_t workspace_bytes, void* stream) {
    return run_gemm(w, false, sk::PRO_RMSNORM, x, nullptr, 0, xt, gamma, eps, m, y, nullptr,
                    nullptr, nullptr, workspace, workspace_bytes, stream, true);
}

SK_EXPORT sk_status sk_gemm_fused_swiglu(const sk_weight* w, const void* gate, const void* up,
                                         int64_t ld, int xt, int m, float* y, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    return run_gemm(w, false, sk::PRO_SWIGLU, gate, up, ld, xt, nullptr, 0.0f, m, y, nullptr,
                    nullptr, nullptr, workspace, workspace_bytes, stream, true);
}

SK_EXPORT sk_status sk_gemm_experts(const sk_weight* bank, int rows_per_expert,
                                    const int32_t* experts, int n_list, const void* x, int xt,
                                    int m, float* y, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    sk_status s = check_weight(bank);
    if (s != SK_OK) return s;
    if (!experts) return SK_ERR_NULL;
    if (rows_per_expert < 16 || rows_per_expert % 16 != 0 || bank->n % rows_per_expert != 0)
        return SK_ERR_SHAPE;
    if (n_list < 1 || (int64_t)n_list * rows_per_expert > (1 << 24)) return SK_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(experts) & 3u) != 0) return SK_ERR_ALIGN;
    return run_gemm(bank, bank->format == SK_W6_SYM, sk::PRO_NONE, x, nullptr, 0, xt, nullptr, 0.0f,
                    m, y, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream, true, false,
                    rows_per_expert, experts, n_list);
}

SK_EXPORT sk_status sk_debug_gemm(const sk_weight* w, int prologue, const void* x, const void* x2,
                                  int64_t ld, int xt, const float* gamma, float eps, int m,
                                  float* y, int8_t* q_out, float* sx_out, int32_t* p_out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (prologue < sk::PRO_NONE || prologue > sk::PRO_SWIGLU) return SK_ERR_FORMAT;
    return run_gemm(w, false, prologue, x, x2, ld, xt, gamma, eps, m, y, q_out, sx_out, p_out,
                    workspace, workspace_bytes, stream, true);
}

SK_EXPORT sk_status sk_quantize_rows(const void* x, int xt, int m, int k, int8_t* q, float* sx,
                                     void* stream) {
    if (!x || !q || !sx) return SK_ERR_NULL;
    if (xt != SK_F32 && xt != SK_BF16) return SK_ERR_FORMAT;
    if (m < 1 || m > 8 || k < 16 || k % 16 != 0) return SK_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || (reinterpret_cast<uintptr_t>(sx) & 3u) != 0)
        return SK_ERR_ALIGN;
    return from_hip(sk::launch_quantize(x, xt, m, k, q, sx, static_cast<hipStream_t>(stream)));
}

SK_EXPORT sk_status sk_prologue_rmsnorm(const void* x, int xt, const float* gamma, float eps, int m, int k,
                                        float* h, void* stream) {
    if (!x || !gamma || !h) return SK_ERR_NULL;
    if (xt != SK_F32 && xt != SK_BF16) return SK_ERR_FORMAT;
    if (m < 1 || m > 8 || k < 16 || k % 16 != 0) return SK_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(h)) return SK_ERR_ALIGN;
    return from_hip(sk::launch_prologue(sk::PRO_RMSNORM, x, nullptr, k, xt, gamma, eps, m, k, h,
                                        static_cast<hipStream_t>(stream)));
}

SK_EXPORT sk_status sk_prologue_swiglu(const void* gate, const void* up, int64_t ld, int xt, int m, int k,
                                       float* h, void* stream) {
    if (!gate || !up || !h) return SK_ERR_NULL;
    if (xt != SK_F32 && xt != SK_BF16) return SK_ERR_FORMAT;
    if (m < 1 || m > 8 || k < 16 || k % 16 != 0 || ld < k) return SK_ERR_SHAPE;
    const int esize = (xt == SK_BF16) ? 2 : 4;
    if ((ld * esize) % 16 != 0 || !aligned16(gate) || !aligned16(up) || !aligned16(h)) return SK_ERR_ALIGN;
    return from_hip(sk::launch_prologue(sk::PRO_SWIGLU, gate, up, ld, xt, nullptr, 0.0f, m, k, h,
                                        static_cast<hipStream_t>(stream)));
}

SK_EXPORT sk_status sk_gemm_w4a8_canonical(const sk_weight* w, const void* x, int xt, int m,
                                           float* y, void* workspace, size_t workspace_bytes,
                                           void* stream) {
    return run_gemm(w, false, sk::PRO_NONE, x, nullptr, 0, xt, nullptr, 0.0f, m, y, nullptr,
                    nullptr, nullptr, workspace, workspace_bytes, stream, false, true);
}

SK_EXPORT sk_status sk_gemm_w4a8_canonical_q(const sk_weight* w, const int8_t* q, const float* sx,
                                             int m, float* y, void* workspace, size_t workspace_bytes,
                                             void* stream) {
    if (sx && (reinterpret_cast<uintptr_t>(sx) & 3u) != 0) return SK_ERR_ALIGN;
    return run_gemm(w, false, sk::PRO_QIN, q, sx, 0, SK_F32, nullptr, 0.0f, m, y, nullptr,
                    nullptr, nullptr, workspace, workspace_bytes, stream, false, true);
}

SK_EXPORT sk_status sk_test_repack_on_host(const sk_weight* w, void* host_bytes, int inverse) {
    if (!w || !host_bytes) return SK_ERR_NULL;
    sk_weight tmp = *w;
    tmp.data = host_bytes;
    tmp.layout = SK_LAYOUT_CANONICAL;
    sk_status s = check_weight(&tmp);
    if (s != SK_OK) return s;
    const Geom G = sk::make_geom(w->n, w->k, w->group, w->format);
    return sk::repack_host(static_cast<uint8_t*>(host_bytes), G, inverse != 0) ? SK_OK
                                                                               : SK_ERR_SHAPE;
}

SK_EXPORT sk_status sk_test_gemm_plan(int n, int k, int group, int format, int m, int prologue,
                                      int cus, int64_t* fields) {
    if (!fields) return SK_ERR_NULL;
    if (n < 1 || k < 128 || k % 128 != 0 || group < 16 || 128 % group != 0 || m < 1 || m > 8 ||
        cus < 1 || prologue < 0 || prologue > 2)
        return SK_ERR_SHAPE;
    const Geom G = sk::make_geom(n, k, group, format);
    const sk::Plan p = sk::make_plan(G, m, prologue, cus, 0);
    const int64_t v[15] = {p.S, p.R, p.P, p.TW, p.KW, p.spw, p.KBs, p.KS, p.WPR, (int64_t)p.lds,
                           (int64_t)p.part_floats, p.ept, p.wide ? 1 : 0, p.pipe, p.srem};
    for (int i = 0; i < 15; ++i) fields[i] = v[i];
    return p.ok ? SK_OK : SK_ERR_UNSUPPORTED;
}

SK_EXPORT sk_status sk_test_set_split(int s) {
    if (s < 0 || s > 32) return SK_ERR_SHAPE;
    sk::set_split_override(s);
    return SK_OK;
}

SK_EXPORT sk_status sk_test_set_spin_limit(int polls) {
    if (polls < 0) return SK_ERR_SHAPE;
    g_spin_limit = polls;
    return SK_OK;
}

namespace {

// The streaming-read probe: workgroup b reads 16-byte words [b * per, (b + 1) * per)
// of the buffer, eight loads per thread in flight; words at or past n16 are not read.
__global__ __launch_bounds__(1024) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                           uint32_t* out) {
    constexpr int U = 8;
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b = (int64_t)blockIdx.x * per;
    const int64_t e = b + per < n16 ? b + per : n16;
    uint32_t acc = 0;
    for (int64_t i = b + threadIdx.x; i < e; i += (int64_t)blockDim.x * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + (int64_t)u * blockDim.x;
            v[u] = j < e ? p[j] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) out[0] = acc;
}

}  // namespace

SK_EXPORT sk_status sk_test_stream_read(const void* buf, int64_t bytes, int grid, int threads,
                                        uint32_t* out, void* stream) {
    if (!buf || !out) return SK_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0 || grid < 1 || threads < 64 || threads > 1024 || threads % 64 != 0)
        return SK_ERR_SHAPE;
    if (!aligned16(buf)) return SK_ERR_ALIGN;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3((unsigned)threads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? SK_OK : SK_ERR_HIP;
}

