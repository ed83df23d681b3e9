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
