// sk_gemm.hip -- launch planning and dispatch of the skinny quantized GEMM
// (the kernel itself is in sk_gemm_kernel.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "sk_gemm_kernel.h"

namespace sk {

namespace {

// --------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------

// Production kernels carry no debug-export code; the test hook's calls (any of
// q_out / sx_out / p_out set) run the instances that have it.
KernelFn pick(int fmt, int pro, int xt, int gs, bool dot4, bool dbg, bool wide) {
    switch (fmt) {
        case FMT_W6: return dbg ? pick_kernel_w6_dbg(pro, xt, gs, dot4, wide) : pick_kernel_w6(pro, xt, gs, dot4, wide);
        case FMT_CB: return dbg ? pick_kernel_cb_dbg(pro, xt, gs, dot4, wide) : pick_kernel_cb(pro, xt, gs, dot4, wide);
        default: return dbg ? pick_kernel_w4_dbg(pro, xt, gs, dot4, wide) : pick_kernel_w4(pro, xt, gs, dot4, wide);
    }
}

// Compute units per device, read once per device (a host-side property query).
std::mutex g_mu;
int g_cus[64] = {0};

int g_split_override = 0;

}  // namespace

// ---------------------------------------------------------------------------
// launch planning (pure host logic)
// ---------------------------------------------------------------------------

namespace {

// Waves of a workgroup: TW tile groups x KW waves along k (KW divides the
// slice's KBs super-blocks, or with `uneven` the first KBs % KW k-parts take one
// super-block more).  Each wave walks ceil(tiles / TW) tile steps of its k-part,
// in groups of `pipe` slots (a step's last group padded with slots that load
// nothing); the split with the fewest slots per wave (the longest k-part),
// padding included (the register pipeline's round trips), wins, then the one
// with the fewest real slots per wave, then the one with the fewest tile
// steps (each ends with a workgroup barrier).  Returns the padded slots per wave.
int64_t split_waves(int KBs, int tiles_per_wg, int m, int nwa, int pipe, bool uneven, int& KW, int& TW) {
    KW = 1;
    TW = 1;
    int64_t best_slots = -1, best_real = -1, best_steps = -1;
    for (int kw = 1; kw <= nwa && kw <= KBs; ++kw) {
        if (!uneven && KBs % kw != 0) continue;
        int tw = nwa / kw;
        while (tw > 1 && tw * m * 16 > NT) --tw;      // the epilogue uses one thread per output
        if (tw > tiles_per_wg) tw = tiles_per_wg;
        const int64_t steps = (tiles_per_wg + tw - 1) / tw;
        const int spw = (KBs + kw - 1) / kw;              // the longest k-part
        const int64_t slots = steps * ((spw + pipe - 1) / pipe * pipe);   // padded to whole groups
        const int64_t real = steps * spw;
        if (best_slots < 0 || slots < best_slots || (slots == best_slots && real < best_real) ||
            (slots == best_slots && real == best_real && steps < best_steps)) {
            best_slots = slots;
            best_real = real;
            best_steps = steps;
            KW = kw;
            TW = tw;
        }
    }
    return best_slots;
}

int workgroups_per_slice(int cus, int S, int T) {
    int R = cus / S;
    if (R > T) R = T;
    if (R > kMaxRanges) R = kMaxRanges;
    return R < 1 ? 1 : R;
}

// The plan for a given number of activations per thread (the kernel's register
// budget for the prologue).  An RMSNorm launch also keeps the slice's gamma in LDS.
Plan plan_for(const Geom& G, int m, int cus, int split_override, int ept, int pro) {
    Plan p;
    const int pipe = pipe_of(m == 1 && G.fmt != FMT_CB, G.fmt == FMT_CB);
    const int KB = (int)G.KB;
    const int T = (int)G.T;
    const bool cb = G.fmt == FMT_CB;
    p.WPR = NW / m;                               // waves per activation row
    const int tpr = p.WPR * 64;
    p.ept = ept;
    p.wide = false;
    auto fits = [&](int s) { return (G.k / s) / ept <= (int64_t)tpr; };
    // dynamic LDS of a launch with s slices: q, the tile-epilogue partials of
    // its wave split (two halves of TW tile groups x M x 16 outputs x kwp), for
    // RMSNorm the slice's gamma, and (integer formats) the quantiser's list of
    // chunks to redo
    auto lds_for = [&](int s, int kw, int tw) {
        const size_t KS = (size_t)(G.k / s);
        const size_t red = 2 * 4 * (size_t)tw * m * 16 * red_kwp(kw);
        const size_t gam = (pro == PRO_RMSNORM) ? 4 * KS : 0;     // RMSNorm: the slice's gamma
        if (cb) return 64 + (size_t)m * (2 * KS + 64) + red + gam;   // levels, bf16 q, partials
        const size_t fix = (size_t)kFixCap * kFixStride * 4;         // list of chunks to redo
        return (size_t)m * (KS + 32) + red + gam + fix;
    };
    auto lds_of = [&](int s) {
        const int R = workgroups_per_slice(cus, s, T);
        int kw, tw;
        split_waves(KB / s, (T + R - 1) / R, m, (s > 1) ? NW - 1 : NW, pipe, s > 1, kw, tw);
        return lds_for(s, kw, tw);
    };
    const size_t kLdsMax = 150 * 1024;
    auto valid = [&](int s) { return s >= 1 && s <= SMAX && KB % s == 0 && fits(s) && lds_of(s) <= kLdsMax; };
    int S = 1;
    if (split_override > 0) {
        S = split_override;
    } else if (!valid(1)) {
        // The slice must fit the thread layout and LDS.  Among the K-splits that
        // do, the cheapest by a cost fitted to measured launch times: 4 per
        // weight slot of a wave, 1/2048 per activation a workgroup quantises
        // (M * KS) and 1/16 per (tile, slice, row) partial a workgroup's merges
        // read (tiles per workgroup * S * M), plus 24 slots when the slices of
        // a range cannot share an XCD (R not a multiple of 8: their exchange
        // then takes device-scope round trips, about 3 us more per launch);
        // ties: fewer slices.
        int64_t best = -1;
        for (int s = 2; s <= SMAX; ++s) {
            if (!valid(s)) continue;
            const int R = workgroups_per_slice(cus, s, T);
            const int64_t tpw = (T + R - 1) / R;
            int kw, tw;
            const int64_t slots = split_waves(KB / s, (int)tpw, m, NW - 1, pipe, true, kw, tw);
            // in units of 1/2048
            const int64_t cost = 8192 * slots + (int64_t)m * (G.k / s) + 128 * tpw * s * m +
                                 ((R & 7) ? 8192 * 24 : 0);
            if (best < 0 || cost < best) {
                best = cost;
                S = s;
            }
        }
    }
    p.S = S;
    p.KBs = (S > 0 && KB % S == 0) ? KB / S : 0;
    p.KS = (S > 0) ? (int)(G.k / S) : 0;
    const int R = (S > 0) ? workgroups_per_slice(cus, S, T) : 1;
    p.R = R;
    // with S > 1 one wave is reserved for the exchange
    const int nwa = (S > 1) ? NW - 1 : NW;
    const int64_t slots = split_waves(p.KBs, (T + R - 1) / R, m, nwa, pipe, S > 1, p.KW, p.TW);
    p.pipe = pipe;
    // 4-bit weights without a prologue also have instances with a 4-slot
    // pipeline: taken where its wave split pads fewer slots (e.g. 4 or 12
    // super-blocks per wave, where 5 slots would carry a stand-in in every
    // group); at M >= 2 only for a saving of at least a tenth (the 27B-class
    // gate+up split, 24 slots instead of 25, was measured slower there and
    // faster at M = 1).  The split path's q-input launches keep the same wave
    // split, so their sums stay in the same order.
    if (G.fmt == FMT_W4 && (pro == PRO_NONE || pro == PRO_QIN) && pipe != 4 && S > 0) {
        int kw4 = 1, tw4 = 1;
        const int64_t slots4 = split_waves(p.KBs, (T + R - 1) / R, m, nwa, 4, S > 1, kw4, tw4);
        const bool fewer = (m == 1) ? slots4 < slots : slots4 * 10 <= slots * 9;
        if (fewer && lds_for(S, kw4, tw4) <= kLdsMax) {
            p.KW = kw4;
            p.TW = tw4;
            p.pipe = 4;
        }
    }
    p.spw = p.KW > 0 ? p.KBs / p.KW : 0;
    p.srem = p.KW > 0 ? p.KBs % p.KW : 0;
    p.P = S * R;
    p.ks = cb ? 2 * p.KS + 64 : p.KS + 32;
    // only as many waves per row as the slice needs: the activation work then
    // sits in the waves that start first, and the other waves skip it
    {
        const int need = (p.KS + ept * 64 - 1) / (ept * 64);
        if (need >= 1 && need < p.WPR) p.WPR = need;
    }
    p.kwp = red_kwp(p.KW);
    p.red_half = p.TW * m * 16 * p.kwp;
    p.lds = (S > 0) ? lds_for(S, p.KW, p.TW) : 0;
    p.part_floats = (S > 1) ? (size_t)T * S * m * 16 : 0;
    p.ok = valid(S) && p.KBs >= 1 && p.spw >= 1 && p.P >= 1 && m >= 1 && m <= 8;
    return p;
}

}  // namespace

Plan make_plan(const Geom& G, int m, int pro, int cus, int split_override) {
    const bool cb = G.fmt == FMT_CB;
    const bool dot4 = (m == 1) && !cb;
    // Each thread quantises at most 16 activations of its row (M = 1 on v_dot4,
    // or a prologue), 32 on the MFMA path without a prologue (the codebook
    // included); the wide instances take 24 (v_dot4), 40 (MFMA, integer formats,
    // no prologue, or RMSNorm with 4-bit weights and one K-slice) and are used
    // only where that needs fewer K-slices.  (The split path's PRO_QIN
    // keeps PRO_NONE's plan, so the two compare like for like.)
    if (dot4 && (pro == PRO_NONE || pro == PRO_QIN)) {
        // M = 1 on v_dot4: 16, or 24 in the wide instances where that saves slices
        const Plan p = plan_for(G, m, cus, split_override, 16, pro);
        Plan w = plan_for(G, m, cus, split_override, 24, pro);
        if (w.ok && (!p.ok || w.S < p.S)) {
            w.wide = true;
            return w;
        }
        return p;
    }
    if (dot4 || pro == PRO_SWIGLU || (cb && pro != PRO_NONE)) return plan_for(G, m, cus, split_override, 16, pro);
    if (cb) return plan_for(G, m, cus, split_override, 32, pro);   // no wide codebook instances
    if (pro == PRO_RMSNORM) {
        if (G.fmt != FMT_W4) return plan_for(G, m, cus, split_override, 16, pro);
        const Plan p = plan_for(G, m, cus, split_override, 16, pro);
        if (p.ok && p.S == 1) return p;
        Plan w = plan_for(G, m, cus, split_override, 40, pro);
        if (w.ok && w.S == 1) {
            w.wide = true;
            return w;
        }
        return p;
    }
    const Plan p = plan_for(G, m, cus, split_override, 32, pro);
    Plan w = plan_for(G, m, cus, split_override, 40, pro);
    if (w.ok && (!p.ok || w.S < p.S)) {
        w.wide = true;
        return w;
    }
    return p;
}

void set_split_override(int s) { g_split_override = s; }

namespace {

// The current device's compute-unit count (256 if it cannot be read: the plan
// is then the one a 256-unit part would use, and any launch fails anyway).
int current_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 256;
        g_cus[dev] = v > 0 ? v : 256;
    }
    return g_cus[dev];
}

}  // namespace

Plan gemm_plan(const Geom& G, int m, int pro) {
    return make_plan(G, m, pro, current_cus(), g_split_override);
}

hipError_t launch_gemm(const Geom& G, const GemmCall& c, hipStream_t st) {
    const Plan p = gemm_plan(G, c.m, c.prologue);
    if (!p.ok) return hipErrorInvalidValue;
    if (p.S > 1 && !c.ws) return hipErrorInvalidValue;

    const bool dot4 = (c.m == 1) && G.fmt != FMT_CB;
    const int gs = (int)(G.g / 32);                // 0 for the codebook's G = 16
    const bool dbg = c.q_out || c.sx_out || c.p_out;
    // the plan's pipeline depth is a performance choice: an instance of any
    // depth computes the same sums for the same wave split
    KernelFn fn = c.canon ? pick_kernel_split(c.prologue, c.xt, gs, dot4, p.wide)
                  : (p.pipe == 4 && !dbg && G.fmt == FMT_W4 && c.prologue == PRO_NONE)
                      ? pick_kernel_w4_pipe4(c.xt, gs, dot4, p.wide)
                      : pick(G.fmt, c.prologue, c.xt, gs, dot4, dbg, p.wide);
    if (!fn) return hipErrorInvalidValue;

    KArgs a;
    a.data = c.data;
    a.codebook = c.codebook;
    a.x = c.x;
    a.x2 = c.x2;
    a.ld = c.ld;
    a.gamma = c.gamma;
    a.eps = c.eps;
    a.y = c.y;
    a.q_out = c.q_out;
    a.sx_out = c.sx_out;
    a.p_out = c.p_out;
    a.ws = static_cast<WsHeader*>(c.ws);
    a.part = c.ws ? reinterpret_cast<u64*>(static_cast<uint8_t*>(c.ws) + kWsHeaderBytes) : nullptr;
    a.n = (int)G.n;
    a.k = (int)G.k;
    a.m = c.m;
    a.m_magic = (65536 + c.m - 1) / c.m;
    a.kwp = p.kwp;
    a.red_half = p.red_half;
    a.T = (int)G.T;
    a.KB = (int)G.KB;
    a.kg = (int)G.kg;
    a.tile_full = G.tile_full;
    a.sbf = (int)(TILE_ROWS * G.sb_row);
    a.swo = (int)(TILE_ROWS * G.wsb_row);
    {
        const int nr = (int)(G.n % TILE_ROWS);
        const int ng = (int)(128 / G.g);
        a.nr_last = nr ? nr : TILE_ROWS;
        a.t_rag = nr ? (int)G.T - 1 : -1;
        a.rag_w = (int64_t)(G.T - 1) * G.tile_full;
        a.rag_s = a.rag_w + (int64_t)G.KB * a.nr_last * G.wsb_row;
        a.rag_sbw = (int)(a.nr_last * G.wsb_row);
        a.rag_sbs = a.nr_last * ng * 4;
    }
    a.S = p.S;
    a.R = p.R;
    a.P = p.P;
    a.TW = p.TW;
    a.KW = p.KW;
    a.spw = p.spw;
    a.srem = p.srem;
    a.KBs = p.KBs;
    a.KS = p.KS;
    a.WPR = p.WPR;
    a.ks = p.ks;
    a.spin_limit = c.spin_limit > 0 ? c.spin_limit : (1 << 20);
    a.tpe = c.rows_per_expert / TILE_ROWS;
    a.tpe_magic = a.tpe > 0 ? (1ull << 40) / (u64)a.tpe + 1 : 0;
    a.n_experts = c.n_experts;
    a.experts = c.experts;
    a.tq = (int)(G.T / p.R);
    a.trem = (int)(G.T % p.R);
    a.jn0 = (a.tq + p.TW - 1) / p.TW;
    a.jn1 = (a.tq + 1 + p.TW - 1) / p.TW;
    const int epc = (c.xt == 1) ? 8 : 4;           // activations per 16-byte chunk
    const int nch = p.ept / epc;                   // chunks per thread
    a.cpr = p.KS / epc;
    a.tpr = p.WPR * 64;
    for (int w = 0; w < NW; ++w) {
        const int m = w / p.WPR, wb = (w % p.WPR) * 64;
        int nw = (m < c.m && a.cpr > wb) ? (a.cpr - wb + a.tpr - 1) / a.tpr : 0;
        if (nw > nch) nw = nch;
        a.wtab[w] = (uint32_t)((w / p.KW) | ((w % p.KW) << 5) | (m << 10) | ((w % p.WPR) << 14) |
                               (nw << 19));
    }

    if (p.lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)p.R, (unsigned)p.S), dim3(NT), p.lds, st, a);
    return hipGetLastError();
}

}  // namespace sk
