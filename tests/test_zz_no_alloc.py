"""The allocation-free GEMM entry point against the regular one.

sk_gemm_w4a8_noalloc runs sk_gemm_w4a8's kernels with the library's fixed
device scratch as the split-K workspace.  Its outputs must equal
sk_gemm_w4a8's bit for bit (same kernels, same launch plan) and match the
oracle, on two calls in a row, the second with a smaller input."""

import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

import gemm_sk_repack_amd as sk  # noqa: E402

from test_gpu_parity import assert_y_close, gpu_weight, sentinel_out, assert_tails_untouched  # noqa: E402


def test_noalloc_matches_regular_entry_point_twice():
    # first call: K split into slices (the scratch holds the exchange and partials);
    # second call: a smaller weight and fewer rows, also split
    cases = [(0, 1040, 17408, 32, 8, True), (0, 272, 12288, 32, 5, False)]
    for fmt, n, k, g, m, bf in cases:
        assert sk.gemm_workspace_size(n, k, g, fmt, m) > 0      # the path that uses the scratch
        w, buf = gpu_weight(fmt, n, k, g, 1300 + n)
        sk.sk_repack_w4a8(w)
        h = S.activations(1301 + m, m, k)
        if bf:
            bits = S.to_bf16_bits(h)
            x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
            h_ref = O.bf16_to_f32(bits)
        else:
            x = torch.from_numpy(h).cuda()
            h_ref = h
        y_na, tail = sentinel_out((m, n), torch.float32)
        sk.sk_gemm_w4a8_noalloc(w, x, y=y_na)
        y_reg = sk.sk_gemm_w4a8(w, x)
        torch.cuda.synchronize()
        assert_tails_untouched(tail)
        assert torch.equal(y_na, y_reg), (n, k, m)
        assert_y_close(y_na.cpu().numpy(), O.reference(fmt, buf, n, k, g, h_ref))


def test_noalloc_rejects_calls_beyond_its_scratch():
    # a 151936-row weight with K = 17408 at M = 8 needs far more than 4 MiB of partials
    w = sk.QuantWeight(torch.empty(0, dtype=torch.uint8, device="cuda"), 151936, 17408, 32, 0)
    w.desc.data = 1 << 20          # never dereferenced: the call is rejected on the host
    w.desc.bytes = sk.weight_bytes(0, 151936, 17408, 32)
    w.desc.layout = sk.SK_LAYOUT_STREAM
    assert sk.gemm_workspace_size(151936, 17408, 32, 0, 8) > (4 << 20)
    x = torch.zeros((8, 17408), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sk.SkError) as e:
        sk.sk_gemm_w4a8_noalloc(w, x)
    assert e.value.status == sk.SK_ERR_WORKSPACE
