// sk_layout.h -- the stream layout of a repacked weight, as index arithmetic
// usable from host and device code.
//
// The weights and their per-group FP32 scales are interleaved in the order the
// GEMM workgroups consume them, so each workgroup streams contiguous memory
// ("Doubling the LLM token rate in ComfyUI", section on optimizing linear
// kernels).  Geometry:
//
//   tile        = 16 consecutive rows n (the last tile may hold fewer, nr)
//   super-block = one tile x 128 consecutive k
//   stream      = tiles in order; inside a tile, super-blocks in k order;
//                 tile t starts at t * (16 * KB * sb_row) bytes.
//
// One super-block of a tile with nr rows (nr = 16 except in the last tile):
//
//   W4 / codebook: nr*64 weight bytes, then nr*ng*4 scale bytes.
//     The weight bytes are 4*nr "lane chunks" of 16 bytes; chunk (h, n) with
//     h = 0..3, n = 0..nr-1 sits at byte (h*nr + n)*16.  Its dword j (0..3)
//     holds the 8 codes of row n at k = 128*kb + 32*j + 8*h + e, e = 0..7, as
//     byte c = u(e=c) | u(e=c+4) << 4, so masking with 0x0F0F0F0F gives codes
//     e = 0..3 and (>>4) & 0x0F0F0F0F gives e = 4..7, one per byte.
//     u = w & 15 (two's complement, as in the canonical bytes) for W4,
//     u = index for the codebook.
//   W6: nr*64 bytes "low plane" laid out exactly as W4 but holding the low 4
//     bits of u = w & 63 (two's complement); then nr*32 bytes "high plane": 8-byte chunk (h, n)
//     at nr*64 + (h*nr + n)*8 with two dwords; dword i covers j0 = 2i and
//     j1 = 2i+1 of chunk (h, n): byte c = hi(j0,c) | hi(j0,c+4) << 2 |
//     hi(j1,c) << 4 | hi(j1,c+4) << 6 with hi = u >> 4 (2 bits).
//   scales: row n's ng = 128/G scales of this super-block at
//     nr*wsb_row + n*ng*4, in group order.
//
// A full tile is thus a sequence of self-contained super-blocks [weights |
// scales].  The last tile, when N % 16 != 0, keeps every 128-bit load aligned
// by storing all KB weight parts first and all KB scale parts after them
// (super-block kb's weights at kb*nr*wsb_row, its scales at
// KB*nr*wsb_row + kb*nr*ssb_row); it is still one contiguous run.
//
// The lane chunk (h, n) is exactly what lane 16*h + n of a wave reads with one
// 128-bit load, and dword j is the B operand of one 16x16x32 int8 MFMA
// (column n, k-octet h) for the 32-k block j.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SK_HD __host__ __device__ inline
#else
#define SK_HD inline
#endif

namespace sk {

constexpr int TILE_ROWS = 16;
constexpr int SB_K = 128;

enum Format : int { FMT_W4 = 0, FMT_CB = 1, FMT_W6 = 2 };

struct Geom {
    int64_t n, k, g;
    int fmt, bits;
    int64_t T;        // number of tiles
    int64_t KB;       // super-blocks per tile
    int64_t ng;       // groups per super-block
    int64_t kg;       // groups per row
    int64_t kb8;      // packed weight bytes per row
    int64_t wsb_row;  // weight bytes per row per super-block (64 or 96)
    int64_t ssb_row;  // scale bytes per row per super-block
    int64_t sb_row;   // wsb_row + ssb_row
    int64_t tile_full;// bytes of a full 16-row tile
    int64_t wbytes;   // canonical packed-weight bytes (scales start here)
    int64_t bytes;    // total bytes
};

SK_HD Geom make_geom(int64_t n, int64_t k, int64_t g, int fmt) {
    Geom G;
    G.n = n; G.k = k; G.g = g; G.fmt = fmt;
    G.bits = (fmt == FMT_W6) ? 6 : 4;
    G.T = (n + TILE_ROWS - 1) / TILE_ROWS;
    G.KB = k / SB_K;
    G.ng = SB_K / g;
    G.kg = k / g;
    G.kb8 = k * G.bits / 8;
    G.wsb_row = SB_K * G.bits / 8;
    G.ssb_row = G.ng * 4;
    G.sb_row = G.wsb_row + G.ssb_row;
    G.tile_full = TILE_ROWS * G.KB * G.sb_row;
    G.wbytes = n * G.kb8;
    G.bytes = G.wbytes + n * G.kg * 4;
    return G;
}

SK_HD int64_t tile_rows(const Geom& G, int64_t t) {
    int64_t r = G.n - t * TILE_ROWS;
    return r < TILE_ROWS ? r : TILE_ROWS;
}

// rows covered by tiles [t0, t1)
SK_HD int64_t rows_in(const Geom& G, int64_t t0, int64_t t1) {
    int64_t e = t1 * TILE_ROWS;
    if (e > G.n) e = G.n;
    return e - t0 * TILE_ROWS;
}

// Offsets, relative to the start of a tile with nr rows, of super-block kb's
// weight part and scale part.
SK_HD int64_t sb_w_rel(const Geom& G, int64_t nr, int64_t kb) {
    return nr == TILE_ROWS ? kb * nr * G.sb_row : kb * nr * G.wsb_row;
}
SK_HD int64_t sb_s_rel(const Geom& G, int64_t nr, int64_t kb) {
    return nr == TILE_ROWS ? kb * nr * G.sb_row + nr * G.wsb_row
                           : G.KB * nr * G.wsb_row + kb * nr * G.ssb_row;
}

// ---------------------------------------------------------------------------
// Phase A of the in-place repack: tile interleave by recursive rotation.
//
// Canonical [W_0 .. W_{T-1} | S_0 .. S_{T-1}] (W_t = the tile's packed weight
// rows, S_t = its scale rows) becomes [W_0 S_0 | W_1 S_1 | ...].  A subproblem
// over tiles [t0, t1) occupies the final byte range of those tiles and holds
// [W_t0..W_{t1-1} | S_t0..S_{t1-1}]; with h = t0 + (t1-t0)/2, rotating the
// middle [W_h..W_{t1-1} | S_t0..S_{h-1}] yields two subproblems of the same
// form.  A rotation of [X | Y] is done as reverse(X), reverse(Y) (pass 0) and
// then reverse(XY) (pass 1).  All units are dwords.
// ---------------------------------------------------------------------------

SK_HD int64_t w_dw(const Geom& G, int64_t t0, int64_t t1) {  // weight dwords of tiles
    return rows_in(G, t0, t1) * G.kb8 / 4;
}
SK_HD int64_t s_dw(const Geom& G, int64_t t0, int64_t t1) {  // scale dwords of tiles
    return rows_in(G, t0, t1) * G.kg;
}

SK_HD int num_levels(const Geom& G) {
    int L = 0;
    int64_t span = G.T;
    while (span > 1) { span = (span + 1) / 2; ++L; }
    return L;
}

// For dword position p and recursion level L, find the rotation that touches p.
// Returns false if p's subproblem at this level has a single tile.  Otherwise
// sets the start of the rotated middle region and the lengths of its first and
// second segments (forward: first = weights of the upper half, second = scales
// of the lower half; inverse: the other way round).
SK_HD bool rotation_at(const Geom& G, int64_t p, int L, bool inverse,
                       int64_t* m0, int64_t* len_a, int64_t* len_b) {
    const int64_t tile_dw = G.tile_full / 4;
    int64_t tau = p / tile_dw;
    if (tau > G.T - 1) tau = G.T - 1;
    int64_t t0 = 0, t1 = G.T;
    for (int l = 0; l < L; ++l) {
        if (t1 - t0 <= 1) return false;
        int64_t h = t0 + (t1 - t0) / 2;
        if (tau < h) t1 = h; else t0 = h;
    }
    if (t1 - t0 <= 1) return false;
    int64_t h = t0 + (t1 - t0) / 2;
    int64_t X = w_dw(G, h, t1);
    int64_t Y = s_dw(G, t0, h);
    *m0 = t0 * tile_dw + w_dw(G, t0, h);
    *len_a = inverse ? Y : X;
    *len_b = inverse ? X : Y;
    return true;
}

// The partner dword that position p swaps with in `pass` (0: reverse the two
// segments separately, 1: reverse their union), or -1 if p does not move or is
// the upper element of its pair (each pair is swapped by its lower position).
SK_HD int64_t rotation_partner(const Geom& G, int64_t p, int L, int pass, bool inverse) {
    int64_t m0, a, b;
    if (!rotation_at(G, p, L, inverse, &m0, &a, &b)) return -1;
    if (p < m0 || p >= m0 + a + b) return -1;
    int64_t i = p - m0;
    if (pass == 0) {
        if (i < a) return (i < a / 2) ? m0 + a - 1 - i : -1;
        int64_t j = i - a;
        return (j < b / 2) ? m0 + a + b - 1 - j : -1;
    }
    return (i < (a + b) / 2) ? m0 + a + b - 1 - i : -1;
}

// ---------------------------------------------------------------------------
// Phase B: the per-tile reorder.  After phase A, tile t's bytes are
// [W_t (nr rows x kb8, row-major) | S_t (nr rows x kg floats, row-major)];
// phase B rewrites them into the super-block layout described above.
// Work is split into units; each unit reads a few source bytes and writes a
// few destination bytes of the same tile.
// ---------------------------------------------------------------------------

// W4/codebook weight unit u = ((n*KB + kb)*4 + h)*4 + j  -> one dword each way.
SK_HD int64_t w4_units(const Geom& G, int64_t nr) { return nr * G.KB * 16; }
SK_HD void w4_unit_pos(const Geom& G, int64_t nr, int64_t u, int64_t* src, int64_t* dst) {
    int64_t j = u & 3, h = (u >> 2) & 3, rest = u >> 4;
    int64_t kb = rest % G.KB, n = rest / G.KB;
    int64_t k0 = kb * SB_K + 32 * j + 8 * h;
    *src = n * G.kb8 + k0 / 2;                                   // canonical row bytes
    *dst = sb_w_rel(G, nr, kb) + (h * nr + n) * 16 + 4 * j;      // lane chunk dword
}
// canonical dword (little-endian bytes b0..b3: codes 2c, 2c+1) -> stream dword
SK_HD uint32_t w4_encode(uint32_t s) {
    uint32_t d = 0;
    for (int c = 0; c < 4; ++c) {
        uint32_t lo = (s >> (8 * ((c) >> 1) + 4 * ((c) & 1))) & 0xF;       // code c
        uint32_t hi = (s >> (8 * ((c + 4) >> 1) + 4 * ((c + 4) & 1))) & 0xF; // code c+4
        d |= (lo | (hi << 4)) << (8 * c);
    }
    return d;
}
SK_HD uint32_t w4_decode(uint32_t d) {
    uint32_t code[8];
    for (int c = 0; c < 4; ++c) {
        code[c] = (d >> (8 * c)) & 0xF;
        code[c + 4] = (d >> (8 * c + 4)) & 0xF;
    }
    uint32_t s = 0;
    for (int c = 0; c < 4; ++c) s |= (code[2 * c] | (code[2 * c + 1] << 4)) << (8 * c);
    return s;
}

// W6 weight unit u = ((n*KB + kb)*4 + h)*2 + i: reads the 2 x 6 canonical bytes
// of the octets j0 = 2i and j1 = 2i+1 and writes low-plane dwords j0, j1 and
// high-plane dword i.
SK_HD int64_t w6_units(const Geom& G, int64_t nr) { return nr * G.KB * 8; }
SK_HD void w6_unit_pos(const Geom& G, int64_t nr, int64_t u, int64_t* src0, int64_t* src1,
                       int64_t* dlo0, int64_t* dlo1, int64_t* dhi) {
    int64_t i = u & 1, h = (u >> 1) & 3, rest = u >> 3;
    int64_t kb = rest % G.KB, n = rest / G.KB;
    int64_t j0 = 2 * i, j1 = 2 * i + 1;
    int64_t k00 = kb * SB_K + 32 * j0 + 8 * h, k01 = kb * SB_K + 32 * j1 + 8 * h;
    *src0 = n * G.kb8 + k00 * 3 / 4;
    *src1 = n * G.kb8 + k01 * 3 / 4;
    int64_t sb = sb_w_rel(G, nr, kb);
    *dlo0 = sb + (h * nr + n) * 16 + 4 * j0;
    *dlo1 = sb + (h * nr + n) * 16 + 4 * j1;
    *dhi = sb + nr * 64 + (h * nr + n) * 8 + 4 * i;
}
// 6 canonical bytes (two 24-bit LE words) -> 8 codes u = w & 63
SK_HD void w6_codes(const uint8_t* b, uint32_t* u) {
    uint32_t w0 = b[0] | (b[1] << 8) | (b[2] << 16);
    uint32_t w1 = b[3] | (b[4] << 8) | (b[5] << 16);
    for (int r = 0; r < 4; ++r) {
        u[r] = (w0 >> (6 * r)) & 0x3F;
        u[r + 4] = (w1 >> (6 * r)) & 0x3F;
    }
}
SK_HD void w6_bytes(const uint32_t* u, uint8_t* b) {
    uint32_t w0 = 0, w1 = 0;
    for (int r = 0; r < 4; ++r) {
        w0 |= (u[r] & 0x3F) << (6 * r);
        w1 |= (u[r + 4] & 0x3F) << (6 * r);
    }
    b[0] = w0 & 0xFF; b[1] = (w0 >> 8) & 0xFF; b[2] = (w0 >> 16) & 0xFF;
    b[3] = w1 & 0xFF; b[4] = (w1 >> 8) & 0xFF; b[5] = (w1 >> 16) & 0xFF;
}
SK_HD uint32_t w6_lo(const uint32_t* u) {
    uint32_t d = 0;
    for (int c = 0; c < 4; ++c) d |= ((u[c] & 0xF) | ((u[c + 4] & 0xF) << 4)) << (8 * c);
    return d;
}
SK_HD uint32_t w6_hi(const uint32_t* u0, const uint32_t* u1) {
    uint32_t d = 0;
    for (int c = 0; c < 4; ++c)
        d |= ((u0[c] >> 4) | ((u0[c + 4] >> 4) << 2) | ((u1[c] >> 4) << 4) | ((u1[c + 4] >> 4) << 6))
             << (8 * c);
    return d;
}
SK_HD void w6_split(uint32_t lo0, uint32_t lo1, uint32_t hi, uint32_t* u0, uint32_t* u1) {
    for (int c = 0; c < 4; ++c) {
        uint32_t hb = (hi >> (8 * c)) & 0xFF;
        u0[c] = ((lo0 >> (8 * c)) & 0xF) | ((hb & 3) << 4);
        u0[c + 4] = ((lo0 >> (8 * c + 4)) & 0xF) | (((hb >> 2) & 3) << 4);
        u1[c] = ((lo1 >> (8 * c)) & 0xF) | (((hb >> 4) & 3) << 4);
        u1[c + 4] = ((lo1 >> (8 * c + 4)) & 0xF) | (((hb >> 6) & 3) << 4);
    }
}

// Scale unit u = (n*KB + kb)*ng + gi -> one float each way.
SK_HD int64_t s_units(const Geom& G, int64_t nr) { return nr * G.KB * G.ng; }
SK_HD void s_unit_pos(const Geom& G, int64_t nr, int64_t u, int64_t* src, int64_t* dst) {
    int64_t gi = u % G.ng, rest = u / G.ng;
    int64_t kb = rest % G.KB, n = rest / G.KB;
    *src = nr * G.kb8 + (n * G.kg + kb * G.ng + gi) * 4;
    *dst = sb_s_rel(G, nr, kb) + (n * G.ng + gi) * 4;
}

}  // namespace sk
