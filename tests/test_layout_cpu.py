"""The repack's index logic on the host: the library's own index functions
(run sequentially by the sk_test_repack_on_host hook) turn canonical bytes
into exactly the stream layout of tests/layout_spec.py, and back."""

import ctypes

import numpy as np
import pytest

import gemm_sk_repack_amd as sk
import oracle as O
import synth as S
from layout_spec import stream_layout

CASES = [
    # fmt, n, k, g
    (0, 16, 128, 32), (0, 1, 128, 32), (0, 5, 256, 64), (0, 17, 256, 32), (0, 40, 512, 128),
    (0, 100, 384, 32), (0, 257, 256, 32), (0, 48, 1024, 32),
    (2, 16, 128, 64), (2, 3, 256, 64), (2, 33, 512, 128), (2, 70, 384, 32),
    (1, 16, 128, 16), (1, 21, 256, 16), (1, 64, 256, 32),
]


def host_repack(fmt, n, k, g, buf, inverse):
    out = np.empty(buf.size + 16, dtype=np.uint8)
    off = (-out.ctypes.data) % 16
    arr = out[off:off + buf.size]
    arr[:] = buf
    desc = sk.SkWeightStruct(n, k, g, fmt, 0, 0, 0, buf.size, 16 if fmt == 1 else None)
    st = sk.LIB.sk_test_repack_on_host(ctypes.byref(desc), arr.ctypes.data, int(inverse))
    assert st == sk.SK_OK, sk.status_string(st)
    return arr.copy()


@pytest.mark.parametrize("fmt,n,k,g", CASES)
def test_host_repack_matches_spec_and_inverts(fmt, n, k, g):
    _, _, buf = S.make_weight(fmt, n, k, g, 1000 + n, 2000 + k)
    spec = stream_layout(fmt, buf, n, k, g)
    assert spec.size == buf.size
    got = host_repack(fmt, n, k, g, buf, False)
    assert np.array_equal(got, spec)
    back = host_repack(fmt, n, k, g, got, True)
    assert np.array_equal(back, buf)


def test_spec_is_a_bijection_of_codes_and_scales():
    # every code and every scale of the canonical buffer appears exactly once,
    # in its own 16-row tile, next to its group's scale
    fmt, n, k, g = 0, 37, 256, 32
    w = np.arange(n * k).reshape(n, k) % 16 - 8
    s = (np.arange(n * (k // g), dtype=np.float32) + 1).reshape(n, k // g)
    buf = S.canonical_buffer(S.pack_w4(w), s)
    lay = stream_layout(fmt, buf, n, k, g)
    # scales: the multiset of floats is unchanged
    G = k // g
    tile_full = 16 * (k // 128) * (64 + 4 * (128 // g))
    found = []
    for t in range(0, n, 16):
        nr = min(16, n - t)
        base = (t // 16) * tile_full
        for kb in range(k // 128):
            if nr == 16:
                sb = base + kb * 16 * (64 + 16)
                sc = lay[sb + 16 * 64: sb + 16 * 80].view(np.float32).reshape(16, 4)
            else:
                sc0 = base + (k // 128) * nr * 64 + kb * nr * 16
                sc = lay[sc0: sc0 + nr * 16].view(np.float32).reshape(nr, 4)
            assert np.array_equal(sc, s[t:t + nr, kb * 4:(kb + 1) * 4])
            found.append(sc.reshape(-1))
    assert np.array_equal(np.sort(np.concatenate(found)), np.sort(s.reshape(-1)))
    assert G == 8


def test_host_hook_validates():
    desc = sk.SkWeightStruct(16, 128, 12, 0, 0, 0, 0, 999, None)
    buf = np.zeros(1024, dtype=np.uint8)
    assert sk.LIB.sk_test_repack_on_host(ctypes.byref(desc), buf.ctypes.data, 0) == sk.SK_ERR_SHAPE
