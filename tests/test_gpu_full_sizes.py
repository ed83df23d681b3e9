"""GPU parity at the full sizes of every GEMM workload that bench.py times.

Each workload runs at its full shape, with bench.py's seeds and its values of M,
so the kernels run in the launch configuration that is timed (the launch plan is a
function of the shape, the format, the prologue and M only).  The oracle
computes the sampled output rows one by one:

* q and sx of every activation row bit-exact (whole rows: they are cheap);
* the per-group int32 partials of the sampled rows bit-exact (integer formats);
* y of the sampled rows within the normalised bound (1e-4);
* the production instance's y bit-identical to the export instance's (the test
  hook runs the same plan with the q/sx/partial exports added).

Workloads: the 9B-class decoder linears at M = 1..8; RMSNorm + QKV and
SwiGLU + down at M = 1, 3, 8; W6 G64 and the G16 codebook at N = 12288 and the
151936-row lm_head at M = 1, 8; the 27B-class layer's linears with bf16
activations at M = 1, 8.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

import gemm_sk_repack_amd as sk  # noqa: E402

from test_gpu_parity import assert_y_close  # noqa: E402
from test_quant_rule_cpu import rule  # noqa: E402


def sample_rows(n, seed, count=64):
    """First and last rows of the weight, both sides of the first tile edge, and random rows."""
    edge = [0, 1, 15, 16, n // 2, n - 17, n - 16, n - 1]
    rnd = np.random.default_rng(seed).choice(n, size=count - len(edge), replace=False)
    return np.unique(np.concatenate([np.array(edge), rnd]))


def row_subset(fmt, buf, n, k, g, rows):
    """The canonical buffer of the weight made of rows `rows` only (codes, then scales)."""
    wb = n * k * S.BITS[fmt] // 8
    codes = buf[:wb].reshape(n, -1)[rows]
    sc = buf[wb:].reshape(n, (k // g) * 4)[rows]
    return np.concatenate([codes.reshape(-1), sc.reshape(-1)])


def bench_weight(fmt, n, k, g, cfg, li):
    """Canonical bytes and the repacked device weight, drawn as bench.py draws them."""
    _, _, buf = S.make_weight(fmt, n, k, g, S.seed_of(cfg, li, S.TENSOR_W),
                              S.seed_of(cfg, li, S.TENSOR_S))
    cb = (torch.from_numpy(S.codebook(S.seed_of(cfg, li, S.TENSOR_CB))).cuda()
          if fmt == S.FMT_W4_CODEBOOK else None)
    w = sk.QuantWeight(torch.from_numpy(buf).cuda(), n, k, g, fmt, cb)
    sk.sk_repack_w4a8(w)
    return w, buf


def compare(fmt, buf, n, k, g, rows, h_ref, out, y_pub, cb=None):
    """Checks one call's exports and outputs against the oracle on the sampled rows."""
    y, q, sx, p = out
    torch.cuda.synchronize()
    assert torch.equal(y, y_pub)
    ref = O.reference(fmt, row_subset(fmt, buf, n, k, g, rows), len(rows), k, g, h_ref, cb)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), ref["sx"].view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    idx = torch.from_numpy(rows).cuda()
    if p is not None:
        assert np.array_equal(p.index_select(1, idx).cpu().numpy().astype(np.int64), ref["P"])
    assert_y_close(y.index_select(1, idx).cpu().numpy(), ref)


DECODER = [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096),
           ("down", 4096, 12288)]


@pytest.mark.parametrize("li", range(len(DECODER)), ids=[d[0] for d in DECODER])
def test_decoder_layer_m_sweep(li):
    _, n, k = DECODER[li]
    g = 32
    w, buf = bench_weight(S.FMT_W4, n, k, g, 1, li)
    rows = sample_rows(n, 5000 + li)
    for m in range(1, 9):
        x = S.activations(S.seed_of(1, m, S.TENSOR_X) + k, m, k)
        xd = torch.from_numpy(x).cuda()
        out = sk.sk_debug_gemm(w, sk.PRO_NONE, xd)
        compare(S.FMT_W4, buf, n, k, g, rows, x, out, sk.sk_gemm_w4a8(w, xd))


@pytest.mark.parametrize("m", [1, 3, 8])
def test_rmsnorm_qkv(m):
    n, k, g = 6144, 4096, 32
    w, buf = bench_weight(S.FMT_W4, n, k, g, 3, 0)
    gam = S.gamma(S.seed_of(3, 0, S.TENSOR_GAMMA), k)
    x = S.activations(S.seed_of(3, 0, S.TENSOR_X), m, k)
    xd, gd = torch.from_numpy(x).cuda(), torch.from_numpy(gam).cuda()
    out = sk.sk_debug_gemm(w, sk.PRO_RMSNORM, xd, gamma=gd, eps=1e-6)
    y_pub = sk.sk_gemm_fused_rmsnorm(w, xd, gd, 1e-6)
    compare(S.FMT_W4, buf, n, k, g, sample_rows(n, 5100 + m),
            O.prologue_rmsnorm(x, gam, 1e-6), out, y_pub)


@pytest.mark.parametrize("m", [1, 3, 8])
def test_swiglu_down(m):
    n, k, g = 4096, 12288, 32
    w, buf = bench_weight(S.FMT_W4, n, k, g, 3, 1)
    gu = np.concatenate([S.activations(S.seed_of(3, 1, S.TENSOR_GATE), m, k),
                         S.activations(S.seed_of(3, 1, S.TENSOR_UP), m, k)], axis=1)
    dev = torch.from_numpy(gu).cuda()
    out = sk.sk_debug_gemm(w, sk.PRO_SWIGLU, dev[:, :k], x2=dev[:, k:])
    y_pub = sk.sk_gemm_fused_swiglu(w, dev[:, :k], dev[:, k:])
    compare(S.FMT_W4, buf, n, k, g, sample_rows(n, 5200 + m),
            O.prologue_swiglu(gu[:, :k], gu[:, k:]), out, y_pub)


FORMATS = [("w6_g64", S.FMT_W6, 12288, 64), ("codebook_g16", S.FMT_W4_CODEBOOK, 12288, 16),
           ("lm_head", S.FMT_W4, 151936, 32)]


@pytest.mark.parametrize("li", range(len(FORMATS)), ids=[f[0] for f in FORMATS])
def test_format_variants(li):
    _, fmt, n, g = FORMATS[li]
    k = 4096
    w, buf = bench_weight(fmt, n, k, g, 4, li)
    cb = w.codebook.cpu().numpy() if fmt == S.FMT_W4_CODEBOOK else None
    rows = sample_rows(n, 5300 + li)
    fn = sk.sk_gemm_w6a8 if fmt == S.FMT_W6 else sk.sk_gemm_w4a8
    for m in (1, 8):
        x = S.activations(S.seed_of(4, li, S.TENSOR_X), m, k)
        xd = torch.from_numpy(x).cuda()
        out = sk.sk_debug_gemm(w, sk.PRO_NONE, xd, want_partials=cb is None)
        compare(fmt, buf, n, k, g, rows, x, out, fn(w, xd), cb)


LAYER_27B = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 34816, 5120),
             ("down", 5120, 17408)]


@pytest.mark.parametrize("li", range(len(LAYER_27B)), ids=[d[0] for d in LAYER_27B])
def test_27b_layer_bf16(li):
    _, n, k = LAYER_27B[li]
    g = 32
    w, buf = bench_weight(S.FMT_W4, n, k, g, 2, li)
    rows = sample_rows(n, 5400 + li)
    for m in (1, 8):
        bits = S.to_bf16_bits(S.activations(S.seed_of(2, li, S.TENSOR_X), m, k))
        xd = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        h = O.bf16_to_f32(bits)
        # bf16 rows hold elements at half the row maximum: their bracketing
        # products round apart, so q checks the corrected-quotient branch too
        assert rule(h, O.quantize_rows(h)[1])[1].any()
        out = sk.sk_debug_gemm(w, sk.PRO_NONE, xd)
        compare(S.FMT_W4, buf, n, k, g, rows, h, out, sk.sk_gemm_w4a8(w, xd))
