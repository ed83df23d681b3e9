"""The C ABI on a machine without a GPU: the library loads, exports every
declared symbol, and rejects bad calls on the host with the documented codes
(validation runs before any HIP call, so these never touch a device)."""

import ctypes
import os
import re

import numpy as np
import pytest

import gemm_sk_repack_amd as sk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced


def declared_symbols():
    names = []
    for h in ("sk_repack.h", "sk_repack_test.h", "sk_attention.h", "sk_mtp.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        names += re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(sk_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    decl = declared_symbols()
    assert set(decl) == set(sk.EXPORTS), decl
    for name in decl:
        assert hasattr(sk.LIB, name), name


def test_status_strings():
    for s in range(9):
        assert sk.status_string(s)
    assert sk.status_string(99) == "unknown status"


def W(n=64, k=256, g=32, fmt=0, layout=0, data=FAKE, nbytes=None, cb=None, reserved=0):
    if nbytes is None:
        nbytes = sk.weight_bytes(fmt, n, k, g)
    return sk.SkWeightStruct(n, k, g, fmt, layout, reserved, data, nbytes, cb)


def gemm(w, x=FAKE, xt=0, m=1, y=FAKE, ws=None, wsb=0):
    return sk.LIB.sk_gemm_w4a8(ctypes.byref(w), x, xt, m, y, ws, wsb, None)


def test_null_pointers():
    assert sk.LIB.sk_repack_w4a8(None, None) == sk.SK_ERR_NULL
    assert sk.LIB.sk_repack_w4a8(ctypes.byref(W(data=None)), None) == sk.SK_ERR_NULL
    assert gemm(W(layout=1), x=None) == sk.SK_ERR_NULL
    assert gemm(W(layout=1), y=None) == sk.SK_ERR_NULL
    w = W(layout=1)
    assert sk.LIB.sk_gemm_fused_rmsnorm(ctypes.byref(w), FAKE, 0, None, 1e-6, 1, FAKE, None, 0, None) \
        == sk.SK_ERR_NULL
    assert sk.LIB.sk_gemm_fused_swiglu(ctypes.byref(w), FAKE, None, 256, 0, 1, FAKE, None, 0, None) \
        == sk.SK_ERR_NULL


def test_format_errors():
    assert gemm(W(fmt=7, nbytes=1)) == sk.SK_ERR_FORMAT
    assert gemm(W(layout=1), xt=5) == sk.SK_ERR_FORMAT
    # codebook format needs a codebook; other formats must not have one
    assert gemm(W(fmt=1, layout=1)) == sk.SK_ERR_FORMAT
    assert gemm(W(fmt=0, layout=1, cb=FAKE)) == sk.SK_ERR_FORMAT
    # entry point / format mismatch
    w6 = W(fmt=2, g=64, layout=1)
    assert gemm(w6) == sk.SK_ERR_FORMAT
    w4 = W(layout=1)
    assert sk.LIB.sk_gemm_w6a8(ctypes.byref(w4), FAKE, 0, 1, FAKE, None, 0, None) == sk.SK_ERR_FORMAT
    assert gemm(W(reserved=1, layout=1)) == sk.SK_ERR_FORMAT


@pytest.mark.parametrize("k,g,fmt", [(48, 12, 0), (40, 8, 0), (48, 16, 2), (64, 8, 2), (64, 2, 0)])
def test_page_shape_rules_rejected(k, g, fmt):
    assert gemm(W(k=k, g=g, fmt=fmt, layout=1)) == sk.SK_ERR_SHAPE


def test_shape_errors():
    assert gemm(W(layout=1), m=0) == sk.SK_ERR_SHAPE
    assert gemm(W(layout=1), m=9) == sk.SK_ERR_SHAPE
    assert gemm(W(n=0, layout=1)) == sk.SK_ERR_SHAPE
    assert gemm(W(layout=1, nbytes=12345)) == sk.SK_ERR_SHAPE
    w = W(layout=1)
    assert sk.LIB.sk_gemm_fused_swiglu(ctypes.byref(w), FAKE, FAKE, 255, 0, 1, FAKE, None, 0, None) \
        == sk.SK_ERR_SHAPE


def test_align_errors():
    assert gemm(W(layout=1, data=FAKE + 8)) == sk.SK_ERR_ALIGN
    assert gemm(W(layout=1), x=FAKE + 4) == sk.SK_ERR_ALIGN
    assert gemm(W(layout=1), y=FAKE + 4) == sk.SK_ERR_ALIGN
    w = W(layout=1)
    # ld * 4 bytes must be a multiple of 16
    assert sk.LIB.sk_gemm_fused_swiglu(ctypes.byref(w), FAKE, FAKE, 258, 0, 1, FAKE, None, 0, None) \
        == sk.SK_ERR_ALIGN


def test_layout_errors():
    assert gemm(W(layout=0)) == sk.SK_ERR_LAYOUT                     # not repacked
    assert sk.LIB.sk_repack_w4a8(ctypes.byref(W(layout=1)), None) == sk.SK_ERR_LAYOUT
    assert sk.LIB.sk_unrepack_w4a8(ctypes.byref(W(layout=0)), None) == sk.SK_ERR_LAYOUT
    assert gemm(W(layout=5)) == sk.SK_ERR_LAYOUT


def test_backend_restrictions():
    # allowed by the page's rules, not by this backend
    assert gemm(W(k=48, g=16, layout=1)) == sk.SK_ERR_UNSUPPORTED        # K % 128
    assert gemm(W(k=256, g=16, layout=1)) == sk.SK_ERR_UNSUPPORTED       # W4 sym G=16
    assert gemm(W(k=256, g=8, layout=1)) == sk.SK_ERR_UNSUPPORTED        # G < 16
    assert gemm(W(k=20480, g=32, layout=1)) == sk.SK_ERR_UNSUPPORTED     # K too large
    # the codebook GEMM has a launch plan for every supported group size
    for g in (16, 32, 64, 128):
        for m in (1, 8):
            assert sk.gemm_plan(12288, 4096, g, sk.SK_W4_CODEBOOK, m)["status"] == sk.SK_OK


def test_expert_bank_validation():
    """The expert list is a device array read by the kernel: the host checks the
    pointer, its alignment, rows_per_expert and the list length, not the ids."""
    ex = sk.LIB.sk_gemm_experts
    ids = FAKE
    bank = W(n=512, layout=1)                       # 4 experts of 128 rows

    def call(b=bank, rows=128, e=ids, nl=2, x=FAKE, m=1):
        return ex(ctypes.byref(b), rows, e, nl, x, 0, m, FAKE, None, 0, None)
    assert call(e=None) == sk.SK_ERR_NULL
    assert call(rows=100) == sk.SK_ERR_SHAPE
    assert call(rows=96) == sk.SK_ERR_SHAPE
    assert call(nl=0) == sk.SK_ERR_SHAPE
    assert call(nl=(1 << 24) // 128 + 1) == sk.SK_ERR_SHAPE
    assert call(m=9) == sk.SK_ERR_SHAPE
    assert call(e=FAKE + 2) == sk.SK_ERR_ALIGN
    assert call(b=W(n=512, layout=0)) == sk.SK_ERR_LAYOUT
    assert call(x=FAKE + 4) == sk.SK_ERR_ALIGN


def test_workspace_size_and_validation():
    """Launches that split K need a caller-owned workspace; the size query and
    the checks are host arithmetic."""
    size = sk.gemm_workspace_size
    # K = 4096 at M = 1 runs in one slice: no workspace
    assert size(6144, 4096, 32, 0, 1) == 0
    # the 27B-class down projection at M = 8 splits K
    plan = sk.gemm_plan(5120, 17408, 32, 0, 8)
    assert plan["S"] > 1
    need = size(5120, 17408, 32, 0, 8)
    assert need == 16384 + plan["part_floats"] * 8
    assert need == 16384 + 320 * plan["S"] * 8 * 128
    w = W(n=5120, k=17408, layout=1)
    assert gemm(w, m=8) == sk.SK_ERR_WORKSPACE                       # missing
    assert gemm(w, m=8, ws=FAKE, wsb=need - 256) == sk.SK_ERR_WORKSPACE   # too small
    assert gemm(w, m=8, ws=FAKE + 16, wsb=need) == sk.SK_ERR_WORKSPACE   # not 256-byte aligned
    # query errors
    out = ctypes.c_size_t()
    f = sk.LIB.sk_gemm_workspace_size
    assert f(64, 256, 32, 0, 1, 0, None) == sk.SK_ERR_NULL
    assert f(64, 256, 32, 9, 1, 0, ctypes.byref(out)) == sk.SK_ERR_FORMAT
    assert f(64, 256, 32, 0, 1, 5, ctypes.byref(out)) == sk.SK_ERR_FORMAT
    assert f(64, 256, 32, 0, 9, 0, ctypes.byref(out)) == sk.SK_ERR_SHAPE
    assert f(64, 48, 12, 0, 1, 0, ctypes.byref(out)) == sk.SK_ERR_SHAPE
    assert f(64, 20480, 32, 0, 1, 0, ctypes.byref(out)) == sk.SK_ERR_UNSUPPORTED


def test_split_path_validation():
    q = sk.LIB.sk_quantize_rows
    assert q(None, 0, 1, 256, FAKE, FAKE, None) == sk.SK_ERR_NULL
    assert q(FAKE, 0, 1, 256, FAKE, None, None) == sk.SK_ERR_NULL
    assert q(FAKE, 5, 1, 256, FAKE, FAKE, None) == sk.SK_ERR_FORMAT
    assert q(FAKE, 0, 0, 256, FAKE, FAKE, None) == sk.SK_ERR_SHAPE
    assert q(FAKE, 0, 9, 256, FAKE, FAKE, None) == sk.SK_ERR_SHAPE
    assert q(FAKE, 0, 1, 24, FAKE, FAKE, None) == sk.SK_ERR_SHAPE
    assert q(FAKE + 4, 0, 1, 256, FAKE, FAKE, None) == sk.SK_ERR_ALIGN
    assert q(FAKE, 0, 1, 256, FAKE, FAKE + 2, None) == sk.SK_ERR_ALIGN
    can = sk.LIB.sk_gemm_w4a8_canonical
    assert can(ctypes.byref(W(layout=1)), FAKE, 0, 1, FAKE, None, 0, None) == sk.SK_ERR_LAYOUT
    assert can(ctypes.byref(W(fmt=2, g=64, layout=0)), FAKE, 0, 1, FAKE, None, 0, None) == sk.SK_ERR_FORMAT
    assert can(ctypes.byref(W(layout=0)), None, 0, 1, FAKE, None, 0, None) == sk.SK_ERR_NULL
    cq = sk.LIB.sk_gemm_w4a8_canonical_q
    assert cq(ctypes.byref(W(layout=0)), FAKE, None, 1, FAKE, None, 0, None) == sk.SK_ERR_NULL
    assert cq(ctypes.byref(W(layout=0)), FAKE, FAKE + 2, 1, FAKE, None, 0, None) == sk.SK_ERR_ALIGN
    assert cq(ctypes.byref(W(layout=1)), FAKE, FAKE, 1, FAKE, None, 0, None) == sk.SK_ERR_LAYOUT


def test_prologue_launch_validation():
    r = sk.LIB.sk_prologue_rmsnorm
    assert r(None, 0, FAKE, 1e-6, 1, 256, FAKE, None) == sk.SK_ERR_NULL
    assert r(FAKE, 0, None, 1e-6, 1, 256, FAKE, None) == sk.SK_ERR_NULL
    assert r(FAKE, 0, FAKE, 1e-6, 1, 256, None, None) == sk.SK_ERR_NULL
    assert r(FAKE, 7, FAKE, 1e-6, 1, 256, FAKE, None) == sk.SK_ERR_FORMAT
    assert r(FAKE, 0, FAKE, 1e-6, 0, 256, FAKE, None) == sk.SK_ERR_SHAPE
    assert r(FAKE, 0, FAKE, 1e-6, 9, 256, FAKE, None) == sk.SK_ERR_SHAPE
    assert r(FAKE, 0, FAKE, 1e-6, 1, 24, FAKE, None) == sk.SK_ERR_SHAPE
    assert r(FAKE + 4, 0, FAKE, 1e-6, 1, 256, FAKE, None) == sk.SK_ERR_ALIGN
    assert r(FAKE, 0, FAKE + 8, 1e-6, 1, 256, FAKE, None) == sk.SK_ERR_ALIGN
    assert r(FAKE, 0, FAKE, 1e-6, 1, 256, FAKE + 4, None) == sk.SK_ERR_ALIGN
    sw = sk.LIB.sk_prologue_swiglu
    assert sw(None, FAKE, 256, 0, 1, 256, FAKE, None) == sk.SK_ERR_NULL
    assert sw(FAKE, None, 256, 0, 1, 256, FAKE, None) == sk.SK_ERR_NULL
    assert sw(FAKE, FAKE, 256, 0, 1, 256, None, None) == sk.SK_ERR_NULL
    assert sw(FAKE, FAKE, 256, 3, 1, 256, FAKE, None) == sk.SK_ERR_FORMAT
    assert sw(FAKE, FAKE, 255, 0, 1, 256, FAKE, None) == sk.SK_ERR_SHAPE          # ld < K
    assert sw(FAKE, FAKE, 256, 0, 9, 256, FAKE, None) == sk.SK_ERR_SHAPE
    assert sw(FAKE, FAKE, 260, 1, 1, 256, FAKE, None) == sk.SK_ERR_ALIGN          # 520-byte rows
    assert sw(FAKE + 4, FAKE, 256, 0, 1, 256, FAKE, None) == sk.SK_ERR_ALIGN


def test_failed_call_leaves_descriptor_unchanged():
    w = W(layout=0, data=FAKE + 8)
    assert sk.LIB.sk_repack_w4a8(ctypes.byref(w), None) == sk.SK_ERR_ALIGN
    assert w.layout == 0


def test_stream_read_probe_validation():
    """The probe's checks run on the host before any launch (no GPU needed)."""
    f = sk.LIB.sk_test_stream_read
    fake = 1 << 20                                     # never dereferenced: every call is rejected
    assert f(None, 1024, 256, 256, fake, None) == sk.SK_ERR_NULL
    assert f(fake, 1024, 256, 256, None, None) == sk.SK_ERR_NULL
    assert f(fake, 1000, 256, 256, fake, None) == sk.SK_ERR_SHAPE
    assert f(fake, 0, 256, 256, fake, None) == sk.SK_ERR_SHAPE
    assert f(fake, 1024, 0, 256, fake, None) == sk.SK_ERR_SHAPE
    assert f(fake, 1024, 256, 96, fake, None) == sk.SK_ERR_SHAPE
    assert f(fake, 1024, 256, 2048, fake, None) == sk.SK_ERR_SHAPE
    assert f(fake + 4, 1024, 256, 256, fake, None) == sk.SK_ERR_ALIGN
