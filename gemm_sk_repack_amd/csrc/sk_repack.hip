// sk_repack.hip -- one-time, in-place repack of a canonical weight buffer into
// the stream layout of sk_layout.h, and its inverse.
//
// The re-layout happens once per model load, in device memory, without extra
// memory ("Doubling the LLM token rate in ComfyUI", section on optimizing
// linear kernels).  Two phases, both in place:
//   A. tile interleave: [all weight rows | all scale rows] -> per 16-row tile
//      [weight rows | scale rows], by recursive rotations; each rotation is
//      two passes of disjoint dword swaps (reverse both parts, then reverse
//      their union), so every pass is embarrassingly parallel;
//   B. per-tile reorder: one 1024-thread workgroup per tile reads the whole
//      tile into registers, waits until every read has completed, then writes
//      the tile back in super-block order (re-encoding the codes).
#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "sk_internal.h"
#include "sk_layout.h"

namespace sk {

namespace {

constexpr int kReorderThreads = 1024;
// Register budget of phase B: weight units per thread (a W6 unit holds three
// dwords, a W4 unit one) and scale units per thread.
template <int FMT> constexpr int max_w_units() { return FMT == FMT_W6 ? 20 : 40; }
constexpr int kMaxSUnits = 24;

__global__ __launch_bounds__(256) void rotate_pass_kernel(uint32_t* data, Geom G, int L,
                                                          int pass, int inverse, int64_t ndw) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < ndw; p += stride) {
        int64_t q = rotation_partner(G, p, L, pass, inverse != 0);
        if (q >= 0) {
            uint32_t a = data[p];
            uint32_t b = data[q];
            data[p] = b;
            data[q] = a;
        }
    }
}

__device__ inline uint16_t ld16(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }
__device__ inline void st16(uint8_t* p, uint16_t v) { *reinterpret_cast<uint16_t*>(p) = v; }
__device__ inline uint32_t ld32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ inline void st32(uint8_t* p, uint32_t v) { *reinterpret_cast<uint32_t*>(p) = v; }

// All loads of the tile must have landed in registers before any store of the
// same tile is issued by any thread of the workgroup.
__device__ inline void wait_loads_then_barrier() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

template <int FMT, bool INV>
__global__ __launch_bounds__(kReorderThreads) void tile_reorder_kernel(uint8_t* data, Geom G) {
    const int64_t t = blockIdx.x;
    const int64_t nr = tile_rows(G, t);
    uint8_t* tb = data + t * G.tile_full;
    const int tid = threadIdx.x;

    constexpr int kMaxWUnits = max_w_units<FMT>();
    uint32_t wr[kMaxWUnits][FMT == FMT_W6 ? 3 : 1];
    uint32_t sr[kMaxSUnits];

    // ---- read phase ----
    if (FMT == FMT_W6) {
        const int64_t U = w6_units(G, nr);
#pragma unroll
        for (int r = 0; r < kMaxWUnits; ++r) {
            int64_t u = tid + (int64_t)r * kReorderThreads;
            if (u < U) {
                int64_t s0, s1, d0, d1, dh;
                w6_unit_pos(G, nr, u, &s0, &s1, &d0, &d1, &dh);
                if (!INV) {
                    uint8_t b0[6], b1[6];
                    for (int c = 0; c < 3; ++c) {
                        uint16_t v0 = ld16(tb + s0 + 2 * c), v1 = ld16(tb + s1 + 2 * c);
                        b0[2 * c] = v0 & 0xFF; b0[2 * c + 1] = v0 >> 8;
                        b1[2 * c] = v1 & 0xFF; b1[2 * c + 1] = v1 >> 8;
                    }
                    uint32_t u0[8], u1[8];
                    w6_codes(b0, u0);
                    w6_codes(b1, u1);
                    wr[r][0] = w6_lo(u0);
                    wr[r][1] = w6_lo(u1);
                    wr[r][2] = w6_hi(u0, u1);
                } else {
                    uint32_t u0[8], u1[8];
                    w6_split(ld32(tb + d0), ld32(tb + d1), ld32(tb + dh), u0, u1);
                    uint8_t b0[6], b1[6];
                    w6_bytes(u0, b0);
                    w6_bytes(u1, b1);
                    wr[r][0] = b0[0] | (b0[1] << 8) | (b0[2] << 16) | ((uint32_t)b0[3] << 24);
                    wr[r][1] = b0[4] | (b0[5] << 8) | (b1[0] << 16) | ((uint32_t)b1[1] << 24);
                    wr[r][2] = b1[2] | (b1[3] << 8) | (b1[4] << 16) | ((uint32_t)b1[5] << 24);
                }
            }
        }
    } else {
        const int64_t U = w4_units(G, nr);
#pragma unroll
        for (int r = 0; r < kMaxWUnits; ++r) {
            int64_t u = tid + (int64_t)r * kReorderThreads;
            if (u < U) {
                int64_t s, d;
                w4_unit_pos(G, nr, u, &s, &d);
                wr[r][0] = INV ? w4_decode(ld32(tb + d)) : w4_encode(ld32(tb + s));
            }
        }
    }
    {
        const int64_t U = s_units(G, nr);
#pragma unroll
        for (int r = 0; r < kMaxSUnits; ++r) {
            int64_t u = tid + (int64_t)r * kReorderThreads;
            if (u < U) {
                int64_t s, d;
                s_unit_pos(G, nr, u, &s, &d);
                sr[r] = ld32(tb + (INV ? d : s));
            }
        }
    }

    wait_loads_then_barrier();

    // ---- write phase ----
    if (FMT == FMT_W6) {
        const int64_t U = w6_units(G, nr);
#pragma unroll
        for (int r = 0; r < kMaxWUnits; ++r) {
            int64_t u = tid + (int64_t)r * kReorderThreads;
            if (u < U) {
                int64_t s0, s1, d0, d1, dh;
                w6_unit_pos(G, nr, u, &s0, &s1, &d0, &d1, &dh);
                if (!INV) {
                    st32(tb + d0, wr[r][0]);
                    st32(tb + d1, wr[r][1]);
                    st32(tb + dh, wr[r][2]);
                } else {
                    st16(tb + s0, wr[r][0] & 0xFFFF);
                    st16(tb + s0 + 2, wr[r][0] >> 16);
                    st16(tb + s0 + 4, wr[r][1] & 0xFFFF);
                    st16(tb + s1, wr[r][1] >> 16);
                    st16(tb + s1 + 2, wr[r][2] & 0xFFFF);
                    st16(tb + s1 + 4, wr[r][2] >> 16);
                }
            }
        }
    } else {
        const int64_t U = w4_units(G, nr);
#pragma unroll
        for (int r = 0; r < kMaxWUnits; ++r) {
            int64_t u = tid + (int64_t)r * kReorderThreads;
            if (u < U) {
                int64_t s, d;
                w4_unit_pos(G, nr, u, &s, &d);
                st32(tb + (INV ? s : d), wr[r][0]);
            }
        }
    }
    {
        const int64_t U = s_units(G, nr);
#pragma unroll
        for (int r = 0; r < kMaxSUnits; ++r) {
            int64_t u = tid + (int64_t)r * kReorderThreads;
            if (u < U) {
                int64_t s, d;
                s_unit_pos(G, nr, u, &s, &d);
                st32(tb + (INV ? s : d), sr[r]);
            }
        }
    }
}

template <bool INV>
hipError_t launch_reorder(int fmt, uint8_t* data, const Geom& G, hipStream_t st) {
    dim3 grid((unsigned)G.T), block(kReorderThreads);
    if (fmt == FMT_W6)
        hipLaunchKernelGGL((tile_reorder_kernel<FMT_W6, INV>), grid, block, 0, st, data, G);
    else if (fmt == FMT_CB)
        hipLaunchKernelGGL((tile_reorder_kernel<FMT_CB, INV>), grid, block, 0, st, data, G);
    else
        hipLaunchKernelGGL((tile_reorder_kernel<FMT_W4, INV>), grid, block, 0, st, data, G);
    return hipGetLastError();
}

hipError_t launch_rotations(uint8_t* data, const Geom& G, bool inverse, hipStream_t st) {
    const int L = num_levels(G);
    const int64_t ndw = G.bytes / 4;
    int64_t blocks = (ndw + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    for (int step = 0; step < L; ++step) {
        int lvl = inverse ? (L - 1 - step) : step;
        for (int pass = 0; pass < 2; ++pass) {
            hipLaunchKernelGGL(rotate_pass_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                               reinterpret_cast<uint32_t*>(data), G, lvl, pass, inverse ? 1 : 0, ndw);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

bool reorder_fits(const Geom& G) {
    int64_t wu = (G.fmt == FMT_W6) ? w6_units(G, TILE_ROWS) : w4_units(G, TILE_ROWS);
    int64_t wmax = (G.fmt == FMT_W6) ? max_w_units<FMT_W6>() : max_w_units<FMT_W4>();
    int64_t su = s_units(G, TILE_ROWS);
    return wu <= wmax * kReorderThreads && su <= (int64_t)kMaxSUnits * kReorderThreads;
}

hipError_t repack_device(uint8_t* data, const Geom& G, bool inverse, hipStream_t st) {
    hipError_t e;
    if (!inverse) {
        e = launch_rotations(data, G, false, st);
        if (e != hipSuccess) return e;
        return launch_reorder<false>(G.fmt, data, G, st);
    }
    e = launch_reorder<true>(G.fmt, data, G, st);
    if (e != hipSuccess) return e;
    return launch_rotations(data, G, true, st);
}

// Sequential host execution of exactly the same index functions, used only by
// the CPU tests of the layout logic.
bool repack_host(uint8_t* data, const Geom& G, bool inverse) {
    bool in_bounds = true;
    auto rotations = [&](bool inv) {
        const int L = num_levels(G);
        uint32_t* dw = reinterpret_cast<uint32_t*>(data);
        const int64_t ndw = G.bytes / 4;
        for (int step = 0; step < L; ++step) {
            int lvl = inv ? (L - 1 - step) : step;
            for (int pass = 0; pass < 2; ++pass)
                for (int64_t p = 0; p < ndw; ++p) {
                    int64_t q = rotation_partner(G, p, lvl, pass, inv);
                    if (q >= ndw) { in_bounds = false; continue; }
                    if (q >= 0) { uint32_t a = dw[p]; dw[p] = dw[q]; dw[q] = a; }
                }
        }
    };
    auto reorder = [&](bool inv) {
        for (int64_t t = 0; t < G.T; ++t) {
            const int64_t nr = tile_rows(G, t);
            uint8_t* tb = data + t * G.tile_full;
            const int64_t tbytes = nr * G.KB * G.sb_row;
            std::vector<uint8_t> src(tb, tb + tbytes);
            auto ok = [&](int64_t o, int64_t len) {
                if (o < 0 || o + len > tbytes) { in_bounds = false; return false; }
                return true;
            };
            auto r32 = [&](int64_t o) {
                uint32_t v = 0;
                if (ok(o, 4)) memcpy(&v, &src[o], 4);
                return v;
            };
            auto w32 = [&](int64_t o, uint32_t v) { if (ok(o, 4)) memcpy(tb + o, &v, 4); };
            if (G.fmt == FMT_W6) {
                for (int64_t u = 0; u < w6_units(G, nr); ++u) {
                    int64_t s0, s1, d0, d1, dh;
                    w6_unit_pos(G, nr, u, &s0, &s1, &d0, &d1, &dh);
                    uint32_t u0[8], u1[8];
                    if (!ok(s0, 6) || !ok(s1, 6)) continue;
                    if (!inv) {
                        w6_codes(&src[s0], u0);
                        w6_codes(&src[s1], u1);
                        w32(d0, w6_lo(u0)); w32(d1, w6_lo(u1)); w32(dh, w6_hi(u0, u1));
                    } else {
                        w6_split(r32(d0), r32(d1), r32(dh), u0, u1);
                        w6_bytes(u0, tb + s0);
                        w6_bytes(u1, tb + s1);
                    }
                }
            } else {
                for (int64_t u = 0; u < w4_units(G, nr); ++u) {
                    int64_t s, d;
                    w4_unit_pos(G, nr, u, &s, &d);
                    if (!inv) w32(d, w4_encode(r32(s)));
                    else w32(s, w4_decode(r32(d)));
                }
            }
            for (int64_t u = 0; u < s_units(G, nr); ++u) {
                int64_t s, d;
                s_unit_pos(G, nr, u, &s, &d);
                if (!inv) w32(d, r32(s)); else w32(s, r32(d));
            }
        }
    };
    if (!inverse) { rotations(false); reorder(false); }
    else { reorder(true); rotations(true); }
    return in_bounds;
}

}  // namespace sk
