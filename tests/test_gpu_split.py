"""GPU parity of the split path (the canonical-layout GEMM and the separate
quantisation launch), through the C ABI, against the oracle and against the
fused stream-layout path.

Bar: q and sx bit-exact against the oracle; y within the parity bound of the
oracle and bit-identical to the fused path's y (the split path computes the
same int32 partials and adds them in the same order).
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

import gemm_sk_repack_amd as sk  # noqa: E402

from test_gpu_parity import assert_y_close, gpu_weight, to_dev  # noqa: E402


@pytest.mark.parametrize("xt", ["f32", "bf16"])
@pytest.mark.parametrize("m,k", [(1, 1024), (3, 4096), (8, 4096), (8, 12288), (2, 17408)])
def test_quantize_rows_bit_exact(xt, m, k):
    h = S.activations(700 + m + k, m, k)
    h[0, ::7] *= 40.0                          # a wide spread in one row
    if m > 2:
        h[1] = 0.0                             # all-zero row: sx = 0, q = 0
        h[2] = np.float32(0.75)                # constant row
    dev, ref_h = to_dev(h, xt)
    q, sx = sk.sk_quantize_rows(dev)
    torch.cuda.synchronize()
    q_ref, sx_ref = O.quantize_rows(ref_h)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_quantize_rows_ties_take_exact_division():
    # values whose quotient by sx lands on (or next to) half-integers
    k = 1024
    h = np.zeros((2, k), np.float32)
    h[:, 0] = 127.0
    h[:, 1:257] = np.arange(256, dtype=np.float32) * np.float32(0.5) - np.float32(63.75)
    h[1] *= np.float32(1.0000001)
    dev = torch.from_numpy(h).cuda()
    q, sx = sk.sk_quantize_rows(dev)
    torch.cuda.synchronize()
    q_ref, sx_ref = O.quantize_rows(h)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sx.cpu().numpy(), sx_ref)


CASES = [(640, 2048, 32, (1, 2, 8)), (1000, 4096, 64, (1, 8)), (392, 4096, 128, (1, 5)),
         (2048, 12288, 32, (1, 8)), (6144, 4096, 32, (1, 8)), (1040, 5120, 32, (6, 8)),
         (512, 12288, 32, (3,)), (256, 17408, 32, (1,))]


@pytest.mark.parametrize("n,k,g,ms", CASES)
def test_canonical_gemm_matches_stream_path_and_oracle(n, k, g, ms):
    w_can, buf = gpu_weight(0, n, k, g, 900 + n)
    w_str, _ = gpu_weight(0, n, k, g, 900 + n)
    sk.sk_repack_w4a8(w_str)
    for m in ms:
        h = S.activations(910 + m, m, k)
        x = torch.from_numpy(h).cuda()
        y_fused = sk.sk_gemm_w4a8(w_str, x)
        y_can = sk.sk_gemm_w4a8_canonical(w_can, x)
        q, sx = sk.sk_quantize_rows(x)
        y_split = sk.sk_gemm_w4a8_canonical_q(w_can, q, sx)
        torch.cuda.synchronize()
        assert torch.equal(y_can, y_fused), (n, k, g, m)
        assert torch.equal(y_split, y_fused), (n, k, g, m)
        ref = O.reference(0, buf, n, k, g, h)
        assert_y_close(y_split.cpu().numpy(), ref)
    # the canonical bytes are read in place, never modified
    assert np.array_equal(w_can.data.cpu().numpy(), buf)


def test_canonical_gemm_bf16_and_forced_split():
    n, k, g = 512, 4096, 32
    w_can, buf = gpu_weight(0, n, k, g, 931)
    w_str, _ = gpu_weight(0, n, k, g, 931)
    sk.sk_repack_w4a8(w_str)
    h = S.activations(932, 4, k)
    dev, _ = to_dev(h, "bf16")
    assert torch.equal(sk.sk_gemm_w4a8_canonical(w_can, dev), sk.sk_gemm_w4a8(w_str, dev))
    try:
        sk.set_split(4)
        x = torch.from_numpy(h).cuda()
        q, sx = sk.sk_quantize_rows(x)
        y_a = sk.sk_gemm_w4a8(w_str, x)
        y_b = sk.sk_gemm_w4a8_canonical(w_can, x)
        y_c = sk.sk_gemm_w4a8_canonical_q(w_can, q, sx)
        torch.cuda.synchronize()
    finally:
        sk.set_split(0)
    assert torch.equal(y_b, y_a) and torch.equal(y_c, y_a)


def test_split_entry_points_reject_wrong_layout_and_format():
    n, k, g = 256, 1024, 32
    w, _ = gpu_weight(0, n, k, g, 941)
    x = torch.from_numpy(S.activations(942, 1, k)).cuda()
    sk.sk_repack_w4a8(w)                       # stream layout: the canonical entry refuses it
    with pytest.raises(sk.SkError) as e:
        sk.sk_gemm_w4a8_canonical(w, x)
    assert e.value.status == sk.SK_ERR_LAYOUT
    w6, _ = gpu_weight(2, n, k, 64, 943)
    with pytest.raises(sk.SkError) as e:
        sk.sk_gemm_w4a8_canonical(w6, x)
    assert e.value.status == sk.SK_ERR_FORMAT


# ----------------------------------------------------------------------------
# the prologues as launches of their own
# ----------------------------------------------------------------------------

F32 = np.float32


@pytest.mark.parametrize("xt", ["f32", "bf16"])
@pytest.mark.parametrize("m,k", [(1, 4096), (3, 4096), (8, 12288), (2, 17408), (5, 2064)])
def test_prologue_rmsnorm_launch_bit_exact(xt, m, k):
    h = S.activations(800 + m + k, m, k) * F32(2.5)
    h[0, :32] *= F32(300.0)                         # a wide spread inside one row
    x_dev, x = to_dev(h, xt)
    gam = S.gamma(801 + k, k)
    out = sk.sk_prologue_rmsnorm(x_dev, torch.from_numpy(gam).cuda(), 1e-6)
    torch.cuda.synchronize()
    ref = O.prologue_rmsnorm(x, gam, 1e-6)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("xt", ["f32", "bf16"])
@pytest.mark.parametrize("m,k,pad", [(1, 12288, 0), (3, 12288, 16), (8, 4096, 48), (2, 2064, 0)])
def test_prologue_swiglu_launch_bit_exact(xt, m, k, pad):
    gu = np.zeros((m, 2 * k + pad), np.float32)
    gu[:, :k] = S.activations(810 + m, m, k)
    gu[:, k:2 * k] = S.activations(811 + m, m, k)
    gu[:, :64] *= F32(30.0)                         # exp overflow and underflow branches
    dev, vals = to_dev(gu, xt)
    out = sk.sk_prologue_swiglu(dev[:, :k], dev[:, k:2 * k])
    torch.cuda.synchronize()
    ref = O.prologue_swiglu(vals[:, :k], vals[:, k:2 * k])
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("pro", ["rmsnorm", "swiglu"])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_split_prologue_chains_match_oracle(pro, m):
    """prologue launch -> GEMM quantising in its launch (stream layout), and
    prologue launch -> quantisation launch -> canonical-layout GEMM: q and sx
    bit-exact, y within the parity bound, both against the oracle."""
    n, k, g = (384, 4096, 32) if pro == "rmsnorm" else (256, 12288, 32)
    w_can, buf = gpu_weight(0, n, k, g, 820 + m)
    w_str, _ = gpu_weight(0, n, k, g, 820 + m)
    sk.sk_repack_w4a8(w_str)
    if pro == "rmsnorm":
        x_dev, x = to_dev(S.activations(821 + m, m, k) * F32(2.5), "bf16")
        gam = S.gamma(822, k)
        h = sk.sk_prologue_rmsnorm(x_dev, torch.from_numpy(gam).cuda(), 1e-6)
        h_ref = O.prologue_rmsnorm(x, gam, 1e-6)
        y_fused = sk.sk_gemm_fused_rmsnorm(w_str, x_dev, torch.from_numpy(gam).cuda(), 1e-6)
    else:
        gu = np.concatenate([S.activations(823 + m, m, k), S.activations(824 + m, m, k)], axis=1)
        dev, vals = to_dev(np.ascontiguousarray(gu), "f32")
        h = sk.sk_prologue_swiglu(dev[:, :k], dev[:, k:])
        h_ref = O.prologue_swiglu(vals[:, :k], vals[:, k:])
        y_fused = sk.sk_gemm_fused_swiglu(w_str, dev[:, :k], dev[:, k:])
    y_a = sk.sk_gemm_w4a8(w_str, h)
    q, sx = sk.sk_quantize_rows(h)
    y_b = sk.sk_gemm_w4a8_canonical_q(w_can, q, sx)
    torch.cuda.synchronize()
    ref = O.reference(0, buf, n, k, g, h_ref)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), ref["sx"].view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    for y in (y_a, y_b, y_fused):
        assert_y_close(y.cpu().numpy(), ref)
