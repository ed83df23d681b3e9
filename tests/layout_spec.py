"""The stream layout of a repacked weight, written directly from its definition
(numpy, vectorised).  Test infrastructure: the library's repack, on host and on
GPU, must produce exactly these bytes from the canonical buffer.

Definition (16-row tiles, 128-k super-blocks; u = w & 15 for W4, the index for
the codebook, w & 63 for W6, i.e. the canonical two's-complement codes):
  * tile t at t * tile_full bytes; a full tile is KB super-blocks, each
    [weights | scales]; the ragged last tile stores all KB weight parts, then
    all KB scale parts;
  * weight part of super-block kb: lane chunk (h, n) of 16 bytes at
    (h * nr + n) * 16; its dword j holds codes k = 128 kb + 32 j + 8 h + e as
    byte c = u[e=c] & 15 | (u[e=c+4] & 15) << 4;
  * W6 adds a high plane after the low plane: 8-byte chunk (h, n) at
    nr * 64 + (h * nr + n) * 8; dword i, byte c = hi(2i, c) | hi(2i, c+4) << 2 |
    hi(2i+1, c) << 4 | hi(2i+1, c+4) << 6, hi = u >> 4;
  * scale part: row n's 128/G scales at n * (128/G) * 4.
"""

from __future__ import annotations

import numpy as np

import oracle as O


def _codes(fmt, buf, n, k, g):
    vals, s = O.split_canonical(buf, fmt, n, k, g)
    if fmt == 0:
        u = vals & 15
    elif fmt == 1:
        u = vals
    else:
        u = vals & 63
    return u.astype(np.uint8), s


def _weight_part(fmt, u_rows, KB):
    """u_rows [nr, K] -> uint8 [KB, wbytes_per_superblock] for these rows."""
    nr = u_rows.shape[0]
    x = u_rows.reshape(nr, KB, 4, 4, 8)                    # n, kb, j, h, e
    lo = (x[..., 0:4] & 15) | ((x[..., 4:8] & 15) << 4)    # n, kb, j, h, c
    lo = lo.transpose(1, 3, 0, 2, 4).reshape(KB, -1)       # kb, h, n, j, c
    if fmt != 2:
        return lo.astype(np.uint8)
    hi2 = x >> 4                                           # n, kb, j, h, e
    j0, j1 = hi2[:, :, 0::2], hi2[:, :, 1::2]              # n, kb, i, h, e
    hb = (j0[..., 0:4] | (j0[..., 4:8] << 2) | (j1[..., 0:4] << 4) | (j1[..., 4:8] << 6))
    hb = hb.transpose(1, 3, 0, 2, 4).reshape(KB, -1)       # kb, h, n, i, c
    return np.concatenate([lo, hb], axis=1).astype(np.uint8)


def stream_layout(fmt: int, buf: np.ndarray, n: int, k: int, g: int) -> np.ndarray:
    u, s = _codes(fmt, buf, n, k, g)
    KB, ng = k // 128, 128 // g
    out = []
    for t0 in range(0, n, 16):
        rows = slice(t0, min(t0 + 16, n))
        nr = rows.stop - rows.start
        wp = _weight_part(fmt, u[rows], KB)                                    # KB x wbytes
        sp = np.ascontiguousarray(s[rows].reshape(nr, KB, ng).transpose(1, 0, 2))
        sp = sp.view(np.uint8).reshape(KB, -1)                                 # KB x nr*ng*4
        if nr == 16:
            out.append(np.concatenate([wp, sp], axis=1).reshape(-1))
        else:
            out.append(np.concatenate([wp.reshape(-1), sp.reshape(-1)]))
    return np.concatenate(out)
