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
// PRO_QIN: no prologue and no quantisation in the GEMM; x holds the int8 q
// [M][K] and x2 the float sx [M] that a separate quantisation kernel wrote
// (the split, unfused path kept for comparison).
enum Prologue : int { PRO_NONE = 0, PRO_RMSNORM = 1, PRO_SWIGLU = 2, PRO_QIN = 3 };

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
    int spin_limit;        // polls of an exchange slot before computing it locally (0 = default)
    bool canon;            // weight in the canonical [codes | scales] layout (no repack)
    // expert bank: the call's N is n_list experts x rows_per_expert rows, drawn
    // from the bank by `experts` (device ids); rows_per_expert == 0 otherwise
    int rows_per_expert;
    int n_list;
    int n_experts;         // experts in the bank (ids outside [0, n_experts) give NaN rows)
    const int32_t* experts;
    void* ws;              // caller-owned workspace (null when the plan needs none)
};

// Largest K a GEMM call accepts.
constexpr int64_t kMaxGemmK = 17408;
// Largest number of workgroups per K-slice (one arrival counter each).
constexpr int kMaxRanges = 1024;

// Header of the caller-owned GEMM workspace; only launches that split K into
// S > 1 slices touch it.  It must be zero before its first use; every launch
// leaves it ready for the next.  `gen` counts those launches; exchange slots
// and partials carry gen + 1 as their tag, so stale words from earlier calls
// (of any shape) are never taken for fresh ones.  `cnt[r]` counts the slices
// of workgroup range r that have stored their partials; the last to arrive
// resets it and merges.
struct WsHeader {
    uint32_t gen;
    uint32_t done;
    uint32_t pad[62];
    uint32_t cnt[kMaxRanges];
    unsigned long long amax[32 * 8];   // (tag << 32) | float bits, [slice][row]
    unsigned long long ssh[32 * 8];    // (tag << 32) | high half of the double sum of squares
    unsigned long long ssl[32 * 8];    // (tag << 32) | low half
    // the absmax words again, written and read through the L2 of the writer's
    // chiplet (XCD) only: the fast path between slices that share an XCD
    unsigned long long amax_xcd[32 * 8];
};
// Bytes reserved for the header; the tagged split-K partials follow it.
constexpr size_t kWsHeaderBytes = 16384;
static_assert(sizeof(WsHeader) <= kWsHeaderBytes, "workspace header too large");

// How one GEMM call is laid out on the GPU (pure host arithmetic).
struct Plan {
    int S;        // K-slices (a divisor of K/128, at most 32)
    int R;        // workgroups per slice
    int P;        // workgroups = S * R
    int TW, KW;   // waves = TW tile groups x KW waves along k
    int spw;      // super-blocks per wave per tile (the first srem k-parts take one more)
    int srem;
    int KBs;      // super-blocks per slice
    int KS;       // K per slice
    int WPR;      // waves per activation row in the prologue
    int ept;      // activations per thread (16, 24, 32 or 40)
    bool wide;    // the kernel instances with the larger activation budget
    int ks;       // LDS row stride of q
    int kwp;      // k-parts per tile group rounded up to 4, 8 or 16 (tile-epilogue pitch)
    int red_half; // floats per half of the tile-epilogue partials buffer
    int pipe;     // register-pipeline depth the wave split was chosen for
    size_t lds;   // dynamic LDS bytes
    size_t part_floats;  // workspace words (8 bytes) for slice partials
    bool ok;
};

// Workspace bytes a launch with this plan needs (0 when K is not split).
inline size_t workspace_bytes(const Plan& p) {
    return p.S > 1 ? kWsHeaderBytes + p.part_floats * 8 : 0;
}

Plan make_plan(const Geom& G, int m, int pro, int cus, int split_override);
// The plan a call on the current device would use (ok == false if none).
Plan gemm_plan(const Geom& G, int m, int pro);
void set_split_override(int s);
hipError_t launch_gemm(const Geom& G, const GemmCall& c, hipStream_t st);
// Per-row int8 quantisation of x [M][K] into q [M][K] and sx [M] as its own
// launch (the split path); the same arithmetic as inside the GEMM.
hipError_t launch_quantize(const void* x, int xt, int m, int64_t k, int8_t* q, float* sx,
                           hipStream_t st);
hipError_t launch_prologue(int pro, const void* x, const void* x2, int64_t ld, int xt, const float* gamma,
                           float eps, int m, int64_t k, float* h, hipStream_t st);

}  // namespace sk
