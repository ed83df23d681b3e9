// sk_internal.h -- declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sk_layout.h"

namespace sk {

// repack (sk_repack.hip)
bool reorder_fits(const Geom& G);
hipError_t repack_device(uint8_t* data, const Geom& G, bool inverse, hipStream_t st);
// Returns false if any index fell outside the tile or buffer (never expected).
bool repack_host(uint8_t* data, const Geom& G, bool inverse);

// GEMM (sk_gemm.hip)
enum Prologue : int { PRO_NONE = 0, PRO_RMSNORM = 1, PRO_SWIGLU = 2 };

struct GemmCall {
    const uint8_t* data;   // repacked weight
    const float* codebook; // device float[16] or null
    const void* x;         // activations, or the SwiGLU gate
    const void* x2;        // SwiGLU up (else null)
    int64_t ld;            // row stride of x / x2 in elements
    int xt;                // 0 = f32, 1 = bf16
    const float* gamma;    // RMSNorm weight or null
    float eps;
    int prologue;          // Prologue
    int m;                 // 1..8
    float* y;              // [M][N] f32
    int8_t* q_out;         // debug exports (may be null)
    float* sx_out;
    int32_t* p_out;
};

// Largest K a GEMM call accepts (the int8 activations of all M rows live in LDS).
constexpr int64_t kMaxGemmK = 17408;

size_t gemm_lds_bytes(const Geom& G, int m);
hipError_t launch_gemm(const Geom& G, const GemmCall& c, hipStream_t st);

}  // namespace sk
