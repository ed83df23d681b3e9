"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: quantised activations q and scales sx bit-exact, per-group int32
partials P bit-exact, and Y within 1e-4 of the oracle relative to the
magnitude sx * sum_j |s * P| (the natural scale of fp32 accumulation error;
an elementwise relative error is ill-posed where Y sits near 0).
"""

import numpy as np
import pytest
import torch

import oracle as O
import synth as S
from layout_spec import stream_layout

pytestmark = pytest.mark.gpu

import gemm_sk_repack_amd as sk  # noqa: E402

TOL = 1e-4
F32 = np.float32


def gpu_weight(fmt, n, k, g, seed):
    vals, s, buf = S.make_weight(fmt, n, k, g, seed, seed + 1)
    cb = torch.from_numpy(S.codebook(seed + 6)).cuda() if fmt == 1 else None
    t = torch.from_numpy(buf.copy()).cuda()
    return sk.QuantWeight(t, n, k, g, fmt, cb), buf


def to_dev(h, xt):
    """Activations as the device sees them, and the fp32 values the oracle must use."""
    if xt == "bf16":
        bits = S.to_bf16_bits(h)
        dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        return dev, O.bf16_to_f32(bits)
    return torch.from_numpy(h).cuda(), h


def assert_y_close(y, ref, tol=TOL):
    y = y.astype(np.float64)
    err = np.abs(y - ref["Y"])
    mag = ref["mag"]
    zero = mag == 0
    assert np.all(err[zero] == 0)
    rel = err[~zero] / mag[~zero]
    assert rel.size == 0 or rel.max() <= tol, f"max normalised error {rel.max():.3e}"


SENTINEL = 0x5A
TAIL = 4096


def sentinel_out(shape, dtype):
    """A device tensor of `shape` followed by TAIL elements of sentinel bytes,
    so a store past the end of the output shows up."""
    n = int(np.prod(shape))
    buf = torch.empty(n + TAIL, dtype=dtype, device="cuda")
    buf.view(torch.uint8).fill_(SENTINEL)
    return buf[:n].view(shape), buf[n:]


def assert_tails_untouched(*tails):
    for t in tails:
        assert bool((t.view(torch.uint8) == SENTINEL).all()), "a kernel wrote past the end of its output"


def check_call(w, buf, fmt, n, k, g, h_dev, h_ref, m):
    yo, yt = sentinel_out((m, n), torch.float32)
    qo, qt = sentinel_out((m, k), torch.int8)
    so, st = sentinel_out((m,), torch.float32)
    po, pt = sentinel_out((m, n, k // g), torch.int32) if fmt != 1 else (None, None)
    y, q, sx, p = sk.sk_debug_gemm(w, sk.PRO_NONE, h_dev, want_partials=(fmt != 1), y=yo, q=qo, sx=so, p=po)
    torch.cuda.synchronize()
    assert_tails_untouched(yt, qt, st, *([pt] if pt is not None else []))
    cb = w.codebook.cpu().numpy() if fmt == 1 else None
    ref = O.reference(fmt, buf, n, k, g, h_ref, cb)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), ref["sx"].view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    if p is not None:
        assert np.array_equal(p.cpu().numpy().astype(np.int64), ref["P"])
    assert_y_close(y.cpu().numpy(), ref)
    return y, ref


# ----------------------------------------------------------------------------
# repack
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,n,k,g", [
    (0, 1024, 1024, 32), (0, 1000, 512, 32), (0, 17, 256, 64), (0, 5, 128, 128),
    (0, 6144, 4096, 32), (2, 300, 1024, 64), (2, 33, 256, 32), (1, 48, 256, 16),
])
def test_repack_bytes_match_spec_and_invert(fmt, n, k, g):
    w, buf = gpu_weight(fmt, n, k, g, 7 + n)
    sk.sk_repack_w4a8(w)
    assert w.layout == sk.SK_LAYOUT_STREAM
    torch.cuda.synchronize()
    got = w.data.cpu().numpy()
    assert np.array_equal(got, stream_layout(fmt, buf, n, k, g))
    sk.sk_unrepack_w4a8(w)
    torch.cuda.synchronize()
    assert w.layout == sk.SK_LAYOUT_CANONICAL
    assert np.array_equal(w.data.cpu().numpy(), buf)


def test_repack_allocates_nothing():
    w, _ = gpu_weight(0, 4096, 4096, 32, 3)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    sk.sk_repack_w4a8(w)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


# ----------------------------------------------------------------------------
# GEMM parity
# ----------------------------------------------------------------------------

GEMM_CASES = [
    # fmt, n, k, g, ms
    (0, 1024, 1024, 32, (1, 2, 3, 4, 5, 6, 7, 8)),
    (0, 1000, 512, 32, (1, 3, 8)),
    (0, 17, 256, 64, (1, 5)),
    (0, 5, 128, 128, (1, 2)),
    (0, 2048, 4096, 32, (1, 8)),
    (2, 300, 1024, 64, (1, 4, 8)),
    (2, 33, 256, 32, (1, 8)),
    (2, 64, 512, 128, (1, 8)),
    (1, 1024, 1024, 16, (1, 2, 8)),
    (1, 300, 512, 32, (1, 8)),
    (1, 48, 256, 64, (1, 3)),
    (1, 33, 384, 128, (1, 8)),
    (1, 2048, 4096, 16, (1, 8)),
    # the 40-activation instances (K-slices saved at M >= 6 for K = 5120, M = 3 for K = 12288)
    (0, 528, 5120, 32, (6, 8)),
    (2, 272, 5120, 64, (7, 8)),
    (0, 300, 12288, 32, (3,)),
    # M = 1 with 24 activations per thread (K = 17408 in one slice)
    (0, 96, 17408, 32, (1, 2)),
    (2, 48, 17408, 64, (1,)),
]


@pytest.mark.parametrize("fmt,n,k,g,ms", GEMM_CASES)
@pytest.mark.parametrize("xt", ["f32", "bf16"])
def test_gemm_matches_oracle(fmt, n, k, g, ms, xt):
    w, buf = gpu_weight(fmt, n, k, g, 100 + n + k)
    sk.sk_repack_w4a8(w)
    for m in ms:
        h = S.activations(300 + m, m, k)
        h_dev, h_ref = to_dev(h, xt)
        check_call(w, buf, fmt, n, k, g, h_dev, h_ref, m)


@pytest.mark.parametrize("xt", ["f32", "bf16"])
def test_public_entry_points_equal_debug_run(xt):
    """The public entry points run kernel instances built without the debug
    exports; their y must equal the test hook's bit for bit."""
    for fmt, g in ((0, 32), (2, 64), (1, 16), (0, 128)):
        n, k = 640, 2048
        w, buf = gpu_weight(fmt, n, k, g, 11)
        sk.sk_repack_w4a8(w)
        for m in (1, 3, 8):
            x, _ = to_dev(S.activations(12 + m, m, k), xt)
            y_dbg = sk.sk_debug_gemm(w, sk.PRO_NONE, x, want_partials=False)[0]
            y, yt = sentinel_out((m, n), torch.float32)
            (sk.sk_gemm_w6a8 if fmt == 2 else sk.sk_gemm_w4a8)(w, x, y=y)
            torch.cuda.synchronize()
            assert_tails_untouched(yt)
            assert torch.equal(y, y_dbg), (fmt, g, m, xt)


def test_zero_and_constant_rows():
    n, k, g = 256, 1024, 32
    w, buf = gpu_weight(0, n, k, g, 21)
    sk.sk_repack_w4a8(w)
    h = S.activations(22, 4, k)
    h[1] = 0.0
    h[2] = -3.25
    h[3, :] = 0.0
    h[3, 17] = 1e-30
    y, ref = check_call(w, buf, 0, n, k, g, torch.from_numpy(h).cuda(), h, 4)
    assert np.all(y.cpu().numpy()[1] == 0)


def tiny_rows(k):
    """Rows on both sides of the smallest scale the quantiser's bracket and
    corrected quotient take (sx = 2^-100; below it every element goes through IEEE
    division), with exact ties at that scale, scales down into the subnormal range,
    and rows of subnormal h."""
    rng = np.random.default_rng(27)
    base = S.activations(28, 8, k).astype(np.float64)
    base /= np.abs(base).max(axis=1, keepdims=True)
    amx = [127.0 * 2.0 ** -100,         # sx = 2^-100 exactly: the smallest bracket scale
           127.0 * 2.0 ** -100 * 0.75,  # sx just below it: division throughout
           127.0 * 2.0 ** -125,         # a normal sx far below it
           1e-37, 3e-39, 2e-44, 1e-40,  # sx subnormal; the last rows' h are subnormal too
           1e-30]
    h = (base * np.array(amx)[:, None]).astype(F32)
    for r in (0, 1):                    # h = absmax / 2: quotient 63.5 exactly, a tie to even
        h[r, rng.integers(0, k, 24)] = F32(amx[r] / 2.0) * np.where(rng.random(24) < 0.5, F32(1), F32(-1))
    h[5, rng.integers(0, k, 16)] = F32(2.0 ** -149)     # smallest subnormal values
    h[7, ::3] = F32(3e-41)                              # subnormal h in a row of normal scale
    return h


@pytest.mark.parametrize("m", [1, 3, 8])
@pytest.mark.parametrize("xt", ["f32", "bf16"])
def test_tiny_scale_and_subnormal_activations_bit_exact(m, xt):
    """Denormals are not flushed anywhere in the quantiser: q, sx and P stay
    bit-exact at the smallest scale of the bracket path (with exact ties), below it
    (IEEE division), for subnormal scales and for subnormal activations."""
    n, k, g = 272, 2048, 32
    w, buf = gpu_weight(0, n, k, g, 29)
    sk.sk_repack_w4a8(w)
    h = tiny_rows(k)
    rows = {1: [3], 3: [0, 1, 5], 8: list(range(8))}[m]
    h_dev, h_ref = to_dev(np.ascontiguousarray(h[rows]), xt)
    sx_ref = O.quantize_rows(h_ref)[1]
    assert np.any(sx_ref < 2.0 ** -125)
    if m > 1:
        assert np.any(sx_ref == F32(2.0 ** -100)) and np.any((sx_ref < 2.0 ** -100) & (sx_ref > 2.0 ** -101))
    check_call(w, buf, 0, n, k, g, h_dev, h_ref, m)
    q, sx = sk.sk_quantize_rows(h_dev)
    torch.cuda.synchronize()
    q_ref, sx_ref = O.quantize_rows(h_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))


def near_tie_rows(seed, m, k):
    """Rows whose quotients h / sx sit at or a few float32 steps from half-integers."""
    rng = np.random.default_rng(seed)
    amx = rng.uniform(1e-2, 1e2, size=m).astype(F32)
    sx = (amx / F32(127.0)).astype(np.float64)
    n = rng.integers(-127, 127, size=(m, k)).astype(np.float64)
    h = ((n + 0.5) * sx[:, None]).astype(F32)
    steps = rng.integers(-3, 4, size=(m, k))
    for _ in range(3):
        h = np.where(steps > 0, np.nextafter(h, F32(np.inf)), h)
        h = np.where(steps < 0, np.nextafter(h, F32(-np.inf)), h)
        steps = steps - np.sign(steps)
    h[:, 0] = amx
    return h


@pytest.mark.parametrize("m", [1, 3, 8])
def test_near_tie_activations_bit_exact(m):
    """Quotients next to half-integers take the kernels' corrected-quotient branch."""
    n, k, g = 256, 4096, 32
    w, buf = gpu_weight(0, n, k, g, 25)
    sk.sk_repack_w4a8(w)
    h = near_tie_rows(26 + m, m, k)
    check_call(w, buf, 0, n, k, g, torch.from_numpy(h).cuda(), h, m)
    q, sx = sk.sk_quantize_rows(torch.from_numpy(h).cuda())
    torch.cuda.synchronize()
    q_ref, sx_ref = O.quantize_rows(h)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))


def tie_heavy_rows(seed, m, k):
    """Rows whose quotients h / sx sit on half-integers (before sx is rounded)
    at many elements.  Even rows: absmax 254/128 with every other element an odd
    multiple of 1/128 in [1, 2), so 127 h / absmax = (odd) / 2 for about half
    the row (more such chunks than the kernels list per workgroup); odd rows:
    N(0, 1) with about 100 elements set to +-absmax / 2.  Every value is exact
    in bf16."""
    rng = np.random.default_rng(seed)
    h = S.activations(seed + 1, m, k)
    for r in range(m):
        if r % 2 == 0:
            h[r] = rng.uniform(-0.99, 0.99, k).astype(F32)
            h[r, 0] = F32(254.0 / 128.0)
            idx = rng.choice(np.arange(1, k), k // 2, replace=False)
            odd = 2 * rng.integers(64, 127, size=idx.size) + 1            # 129 .. 253
            h[r, idx] = (odd / 128.0 * np.where(rng.random(idx.size) < 0.5, 1, -1)).astype(F32)
        else:
            amx = np.abs(h[r]).max()
            idx = rng.choice(k, 100, replace=False)
            h[r, idx] = (amx / 2.0 * np.where(rng.random(100) < 0.5, 1, -1)).astype(F32)
    return O.bf16_to_f32(S.to_bf16_bits(h))


@pytest.mark.parametrize("xt", ["f32", "bf16"])
@pytest.mark.parametrize("m,split", [(1, 0), (2, 0), (8, 0), (8, 2)])
def test_tie_heavy_rows_production_equals_debug(xt, m, split):
    """Chunks whose codes need the corrected quotient: the production kernels list
    them and redo them after the quantiser (more of them than the list holds are
    redone in place); the debug instances redo every one in place.  q and sx are
    checked against the oracle on the debug run, and the production y must equal
    the debug y bit for bit."""
    n, k, g = 400, 2048, 32
    w, buf = gpu_weight(0, n, k, g, 41)
    sk.sk_repack_w4a8(w)
    h = tie_heavy_rows(42 + m, 8, k)[:m]
    # row 0 alone has more half-integer quotients than one workgroup's list holds
    sx0 = np.float32(np.abs(h[0]).max() / np.float32(127.0))
    quot = h[0].astype(np.float64) / float(sx0)
    assert np.count_nonzero(np.abs(np.abs(quot - np.trunc(quot)) - 0.5) < 1e-4) > 256
    h_dev, h_ref = to_dev(np.ascontiguousarray(h), xt)
    sk.set_split(split)
    try:
        y_dbg, ref = check_call(w, buf, 0, n, k, g, h_dev, h_ref, m)
        y, yt = sentinel_out((m, n), torch.float32)
        ws = sk.Workspace(sk.gemm_workspace_size(n, k, g, sk.SK_W4_SYM, m)) if split else None
        sk.sk_gemm_w4a8(w, h_dev, y=y, workspace=ws)
        torch.cuda.synchronize()
    finally:
        sk.set_split(0)
    assert_tails_untouched(yt)
    assert torch.equal(y, y_dbg), (xt, m, split)


@pytest.mark.parametrize("n,k,m", [(4096, 12288, 1), (6144, 4096, 8), (2048, 12288, 2)])
def test_pipeline_depths_sum_alike(n, k, m):
    """Shapes whose plan takes the 4-slot pipeline with several slots per wave:
    the production instance (4 slots per load group) and the debug instance (the
    default 5) walk the same wave split in different groups, so their y must be
    equal bit for bit; the debug run is checked against the oracle."""
    p = sk.gemm_plan(n, k, 32, sk.SK_W4_SYM, m)
    assert p["pipe"] == 4 and p["spw"] > 1, p
    g = 32
    w, buf = gpu_weight(0, n, k, g, 51 + m)
    sk.sk_repack_w4a8(w)
    h = S.activations(52 + m, m, k)
    h_dev, h_ref = to_dev(h, "bf16")
    y_dbg, ref = check_call(w, buf, 0, n, k, g, h_dev, h_ref, m)
    y, yt = sentinel_out((m, n), torch.float32)
    ws = sk.Workspace(sk.gemm_workspace_size(n, k, g, sk.SK_W4_SYM, m)) if p["S"] > 1 else None
    sk.sk_gemm_w4a8(w, h_dev, y=y, workspace=ws)
    torch.cuda.synchronize()
    assert_tails_untouched(yt)
    assert torch.equal(y, y_dbg), (n, k, m)


def test_rows_do_not_interact_and_runs_repeat():
    n, k, g = 512, 2048, 32
    w, buf = gpu_weight(0, n, k, g, 31)
    sk.sk_repack_w4a8(w)
    x = torch.from_numpy(S.activations(32, 8, k)).cuda()
    y8 = sk.sk_gemm_w4a8(w, x)
    y8b = sk.sk_gemm_w4a8(w, x)
    torch.cuda.synchronize()
    assert torch.equal(y8, y8b)                        # deterministic
    ref = O.reference(0, buf, n, k, g, x.cpu().numpy())
    y8h = y8.cpu().numpy().astype(np.float64)
    worst = 0.0
    for m in range(1, 8):
        # q and the integer partials of a row never depend on M; y may differ in the
        # last bits because M selects the kernel and the K-split (fp32 summation order)
        ym, q, sx, p = sk.sk_debug_gemm(w, sk.PRO_NONE, x[:m].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), ref["q"][:m])
        assert np.array_equal(p.cpu().numpy().astype(np.int64), ref["P"][:m])
        assert_y_close(ym.cpu().numpy(), {"Y": ref["Y"][:m], "mag": ref["mag"][:m]})
        d = np.abs(ym.cpu().numpy().astype(np.float64) - y8h[:m]) / ref["mag"][:m]
        worst = max(worst, float(d.max()))
    # the row-for-row difference of y across M, reported, and bounded by the two
    # calls' own bounds against the oracle
    print(f"max |y(M=m)[i] - y(M=8)[i]| / mag over m = 1..7: {worst:.3e}")
    assert worst <= 2 * TOL


# ----------------------------------------------------------------------------
# fused prologues
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("m", [1, 3, 5, 8])
@pytest.mark.parametrize("fmt,g", [(0, 32), (2, 64)])
@pytest.mark.parametrize("xt", ["f32", "bf16"])
def test_fused_rmsnorm(m, fmt, g, xt):
    n, k = 384, 4096
    w, buf = gpu_weight(fmt, n, k, g, 41)
    sk.sk_repack_w4a8(w)
    x_dev, x = to_dev(S.activations(42 + m, m, k) * F32(2.5), xt)
    gam = S.gamma(43, k)
    eps = 1e-6
    y, q, sx, p = sk.sk_debug_gemm(w, sk.PRO_RMSNORM, x_dev, gamma=torch.from_numpy(gam).cuda(), eps=eps)
    y_pub = sk.sk_gemm_fused_rmsnorm(w, x_dev, torch.from_numpy(gam).cuda(), eps)
    torch.cuda.synchronize()
    h = O.prologue_rmsnorm(x, gam, eps)
    ref = O.reference(fmt, buf, n, k, g, h)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), ref["sx"].view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    assert np.array_equal(p.cpu().numpy().astype(np.int64), ref["P"])
    assert_y_close(y.cpu().numpy(), ref)
    assert torch.equal(y, y_pub)


@pytest.mark.parametrize("m", [2, 6, 7, 8])
@pytest.mark.parametrize("xt", ["f32", "bf16"])
def test_fused_rmsnorm_hidden_5120(m, xt):
    """At hidden 5120 an RMSNorm launch with M >= 6 holds 40 activations per
    thread (gamma kept in LDS) and runs one K-slice; q, sx and P stay bit-exact,
    N ragged."""
    n, k, g = 400, 5120, 32
    plan = sk.gemm_plan(n, k, g, sk.SK_W4_SYM, m, prologue=sk.PRO_RMSNORM)
    if m >= 6:
        assert plan["S"] == 1 and plan["wide"] and plan["ept"] == 40
    w, buf = gpu_weight(0, n, k, g, 44)
    sk.sk_repack_w4a8(w)
    x_dev, x = to_dev(S.activations(45 + m, m, k) * F32(1.5), xt)
    gam = S.gamma(46, k)
    eps = 1e-5
    y, q, sx, p = sk.sk_debug_gemm(w, sk.PRO_RMSNORM, x_dev, gamma=torch.from_numpy(gam).cuda(), eps=eps)
    y_pub = sk.sk_gemm_fused_rmsnorm(w, x_dev, torch.from_numpy(gam).cuda(), eps)
    torch.cuda.synchronize()
    h = O.prologue_rmsnorm(x, gam, eps)
    ref = O.reference(0, buf, n, k, g, h)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), ref["sx"].view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    assert np.array_equal(p.cpu().numpy().astype(np.int64), ref["P"])
    assert_y_close(y.cpu().numpy(), ref)
    assert torch.equal(y, y_pub)


@pytest.mark.parametrize("m", [1, 3, 8])
@pytest.mark.parametrize("xt", ["f32", "bf16"])
def test_fused_swiglu(m, xt):
    n, k, g = 256, 12288, 32
    w, buf = gpu_weight(0, n, k, g, 51)
    sk.sk_repack_w4a8(w)
    gu = np.concatenate([S.activations(52 + m, m, k), S.activations(62 + m, m, k)], axis=1)
    gu[:, :64] *= 30.0                                     # reach the exp overflow branch
    dev, ref_vals = to_dev(np.ascontiguousarray(gu), xt)
    gate, up = dev[:, :k], dev[:, k:]
    y, q, sx, p = sk.sk_debug_gemm(w, sk.PRO_SWIGLU, gate, x2=up)
    y_pub = sk.sk_gemm_fused_swiglu(w, gate, up)
    torch.cuda.synchronize()
    h = O.prologue_swiglu(ref_vals[:, :k], ref_vals[:, k:])
    ref = O.reference(0, buf, n, k, g, h)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), ref["sx"].view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    assert np.array_equal(p.cpu().numpy().astype(np.int64), ref["P"])
    assert_y_close(y.cpu().numpy(), ref)
    assert torch.equal(y, y_pub)


# ----------------------------------------------------------------------------
# full decoder shapes, sampled rows
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,n,k", [("qkv", 6144, 4096), ("o", 4096, 4096),
                                      ("gate_up", 24576, 4096), ("down", 4096, 12288)])
def test_decoder_shapes_sampled(name, n, k):
    g = 32
    w, buf = gpu_weight(0, n, k, g, 1000 + n // 16)
    sk.sk_repack_w4a8(w)
    rows = np.sort(np.random.default_rng(n).choice(n, size=96, replace=False))
    vals, s = O.split_canonical(buf, 0, n, k, g)
    for m in (1, 8):
        x = S.activations(1002 + m, m, k)
        y = sk.sk_gemm_w4a8(w, torch.from_numpy(x).cuda()).cpu().numpy()
        q, sx = O.quantize_rows(x)
        p = O.group_partials(vals[rows], q, g)
        ref = {"Y": O.output(p, s[rows], sx), "mag": O.output_magnitude(p, s[rows], sx)}
        assert_y_close(y[:, rows], ref)


# ----------------------------------------------------------------------------
# K-split variants: cross-slice exchange and last-arriver merge
# ----------------------------------------------------------------------------

@pytest.fixture
def reset_hooks():
    yield
    sk.set_split(0)
    sk.set_spin_limit(0)


def run_prologue(w, pro, k, m, seed):
    """Returns (debug outputs, oracle reference) for one prologue kind."""
    if pro == sk.PRO_SWIGLU:
        gu = np.concatenate([S.activations(seed, m, k), S.activations(seed + 1, m, k)], axis=1)
        dev = torch.from_numpy(np.ascontiguousarray(gu)).cuda()
        out = sk.sk_debug_gemm(w, pro, dev[:, :k], x2=dev[:, k:])
        h = O.prologue_swiglu(gu[:, :k], gu[:, k:])
    elif pro == sk.PRO_RMSNORM:
        x = S.activations(seed, m, k)
        gam = S.gamma(seed + 2, k)
        out = sk.sk_debug_gemm(w, pro, torch.from_numpy(x).cuda(),
                               gamma=torch.from_numpy(gam).cuda(), eps=1e-6)
        h = O.prologue_rmsnorm(x, gam, 1e-6)
    else:
        x = S.activations(seed, m, k)
        out = sk.sk_debug_gemm(w, pro, torch.from_numpy(x).cuda())
        h = x
    torch.cuda.synchronize()
    return out, h


def assert_bit_exact(out, ref):
    y, q, sx, p = out
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), ref["sx"].view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    assert np.array_equal(p.cpu().numpy().astype(np.int64), ref["P"])
    assert_y_close(y.cpu().numpy(), ref)


@pytest.mark.parametrize("split", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("pro", [sk.PRO_NONE, sk.PRO_RMSNORM, sk.PRO_SWIGLU])
def test_forced_split_matches_oracle(split, pro, reset_hooks):
    n, k, g = 520, 4096, 32
    w, buf = gpu_weight(0, n, k, g, 71)
    sk.sk_repack_w4a8(w)
    sk.set_split(split)
    ran = 0
    for m in (1, 3, 8):
        # a forced split must still fit the kernel's register layout
        sk.set_split(0)
        p = sk.gemm_plan(n, k, g, 0, m, prologue=pro)
        sk.set_split(split)
        tpr = (16 // m) * 64
        # the largest budget of activations per thread among the kernel instances
        if m == 1 or pro == sk.PRO_SWIGLU:
            ept = 16
        elif pro == sk.PRO_RMSNORM:
            ept = 32 if split == 1 else 16           # the one-slice RMSNorm instances
        else:
            ept = 40
        if (k // split) // ept > tpr:
            with pytest.raises(sk.SkError):
                run_prologue(w, pro, k, m, 72 + m)
            continue
        ran += 1
        out, h = run_prologue(w, pro, k, m, 72 + m)
        assert_bit_exact(out, O.reference(0, buf, n, k, g, h))
    assert ran >= 1


@pytest.mark.parametrize("pro", [sk.PRO_NONE, sk.PRO_RMSNORM, sk.PRO_SWIGLU])
def test_exchange_local_fallback_is_identical(pro, reset_hooks):
    n, k, g = 1040, 4096, 32
    w, buf = gpu_weight(0, n, k, g, 81)
    sk.sk_repack_w4a8(w)
    sk.set_split(8)
    fast, h = run_prologue(w, pro, k, 8, 82)
    sk.set_spin_limit(1)                      # almost every slot times out -> computed locally
    slow, _ = run_prologue(w, pro, k, 8, 82)
    for a, b in zip(fast, slow):
        assert torch.equal(a, b)
    assert_bit_exact(slow, O.reference(0, buf, n, k, g, h))


def test_back_to_back_calls_in_one_graph(reset_hooks):
    """Replays of one captured graph that mixes launches with and without a
    K-split: the split ones reuse the workspace's exchange slots, arrival
    counters and generation word on every launch, and every replay with new
    activations must still match the oracle."""
    n, k, g = 2048, 4096, 32
    w, buf = gpu_weight(0, n, k, g, 91)
    sk.sk_repack_w4a8(w)
    x = torch.zeros((8, k), dtype=torch.float32, device="cuda")
    ys = [torch.empty((8, n), dtype=torch.float32, device="cuda") for _ in range(4)]
    ws = sk.Workspace(16 << 20)
    splits = [1, 4, 1, 8]
    for sp in splits:
        sk.set_split(sp)
        assert (sk.gemm_workspace_size(n, k, g, 0, 8) > 0) == (sp > 1)
    x.copy_(torch.from_numpy(S.activations(92, 8, k)))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for sp, y in zip(splits, ys):
            sk.set_split(sp)                  # host-side plan choice, fixed at capture
            sk.sk_gemm_w4a8(w, x, y=y, workspace=ws)
    sk.set_split(0)
    for rep in range(4):
        xh = S.activations(93 + rep, 8, k)
        x.copy_(torch.from_numpy(xh))
        # eager calls of other shapes on the same workspace between replays
        sk.set_split(2)
        sk.sk_gemm_w4a8(w, x[:3].contiguous(), workspace=ws)
        sk.set_split(0)
        graph.replay()
        torch.cuda.synchronize()
        ref = O.reference(0, buf, n, k, g, xh)
        for y in ys:
            assert_y_close(y.cpu().numpy(), ref)


def test_graph_replays_after_the_default_workspace_grows(reset_hooks):
    """A graph captured on the binding's default workspace keeps pointing at
    that buffer; an eager call that needs more replaces the default with a
    larger one but never frees the old, so the graph's replays stay correct."""
    n, k, g, m = 1040, 4096, 32, 8
    w, buf = gpu_weight(0, n, k, g, 95)
    sk.sk_repack_w4a8(w)
    x = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    sk.set_split(4)
    sk.sk_gemm_w4a8(w, x, y=y)                      # the default workspace fits it before capture
    old = sk.default_workspace(1)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sk.sk_gemm_w4a8(w, x, y=y)
    # a call that needs more than the default holds now: enough 16-row tiles,
    # split 8 ways at M = 8 (128 * M * S bytes of partials per tile)
    rows = 16 * (old.nbytes // (128 * m * 8) + 1)
    big, _ = gpu_weight(0, rows, k, g, 96)
    sk.sk_repack_w4a8(big)
    sk.set_split(8)
    need = sk.gemm_workspace_size(rows, k, g, 0, m)
    assert need > old.nbytes
    sk.sk_gemm_w4a8(big, torch.from_numpy(S.activations(97, m, k)).cuda())
    assert sk.default_workspace(1) is not old and sk.default_workspace(1).nbytes >= need
    sk.set_split(0)
    for rep in range(3):
        xh = S.activations(98 + rep, m, k)
        x.copy_(torch.from_numpy(xh))
        graph.replay()
        torch.cuda.synchronize()
        assert_y_close(y.cpu().numpy(), O.reference(0, buf, n, k, g, xh))


def test_concurrent_streams_with_own_workspaces(reset_hooks):
    """Two streams run split-K GEMMs at the same time, each with its own
    workspace; both results match the oracle."""
    n, k, g = 1040, 4096, 32
    wa, bufa = gpu_weight(0, n, k, g, 95)
    wb, bufb = gpu_weight(0, n, k, g, 96)
    sk.sk_repack_w4a8(wa)
    sk.sk_repack_w4a8(wb)
    sk.set_split(4)
    xa_h, xb_h = S.activations(97, 8, k), S.activations(98, 5, k)
    xa, xb = torch.from_numpy(xa_h).cuda(), torch.from_numpy(xb_h).cuda()
    wsa, wsb = sk.Workspace(4 << 20), sk.Workspace(4 << 20)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    ya = [torch.empty((8, n), dtype=torch.float32, device="cuda") for _ in range(6)]
    yb = [torch.empty((5, n), dtype=torch.float32, device="cuda") for _ in range(6)]
    for i in range(6):
        sk.sk_gemm_w4a8(wa, xa, y=ya[i], stream=sa, workspace=wsa)
        sk.sk_gemm_w4a8(wb, xb, y=yb[i], stream=sb, workspace=wsb)
    torch.cuda.synchronize()
    ra = O.reference(0, bufa, n, k, g, xa_h)
    rb = O.reference(0, bufb, n, k, g, xb_h)
    for i in range(6):
        assert_y_close(ya[i].cpu().numpy(), ra)
        assert_y_close(yb[i].cpu().numpy(), rb)


@pytest.mark.parametrize("pro", [sk.PRO_RMSNORM, sk.PRO_SWIGLU])
@pytest.mark.parametrize("m", [1, 8])
def test_codebook_with_prologues(pro, m):
    n, k, g = 200, 1024, 16
    w, buf = gpu_weight(1, n, k, g, 81)
    sk.sk_repack_w4a8(w)
    if pro == sk.PRO_SWIGLU:
        gu = np.concatenate([S.activations(82, m, k), S.activations(83, m, k)], axis=1)
        dev = torch.from_numpy(np.ascontiguousarray(gu)).cuda()
        y, q, sx, _ = sk.sk_debug_gemm(w, pro, dev[:, :k], x2=dev[:, k:], want_partials=False)
        y_pub = sk.sk_gemm_fused_swiglu(w, dev[:, :k], dev[:, k:])
        h = O.prologue_swiglu(gu[:, :k], gu[:, k:])
    else:
        x = S.activations(84, m, k)
        gam = S.gamma(85, k)
        xd, gd = torch.from_numpy(x).cuda(), torch.from_numpy(gam).cuda()
        y, q, sx, _ = sk.sk_debug_gemm(w, pro, xd, gamma=gd, eps=1e-6, want_partials=False)
        y_pub = sk.sk_gemm_fused_rmsnorm(w, xd, gd, 1e-6)
        h = O.prologue_rmsnorm(x, gam, 1e-6)
    torch.cuda.synchronize()
    ref = O.reference(1, buf, n, k, g, h, w.codebook.cpu().numpy())
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), ref["sx"].view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    assert_y_close(y.cpu().numpy(), ref)
    assert torch.equal(y, y_pub)


def test_codebook_of_integer_levels_equals_w4():
    """A codebook holding the levels -8..7 is the plain W4 weight (same codes,
    levels u - 8), so its output equals the W4 path's up to fp32 rounding."""
    n, k, g = 256, 2048, 32
    vals, s, buf = S.make_weight(0, n, k, g, 91, 92)
    w4 = sk.QuantWeight(torch.from_numpy(buf.copy()).cuda(), n, k, g, 0)
    # the same values as unsigned indices u = w + 8
    u = (vals + 8).astype(np.uint8)
    cb_buf = S.canonical_buffer(S.pack_u4(u), s)
    cb = torch.arange(-8, 8, dtype=torch.float32).cuda()
    wc = sk.QuantWeight(torch.from_numpy(cb_buf).cuda(), n, k, g, 1, cb)
    sk.sk_repack_w4a8(w4)
    sk.sk_repack_w4a8(wc)
    for m in (1, 8):
        x = torch.from_numpy(S.activations(93 + m, m, k)).cuda()
        y4 = sk.sk_gemm_w4a8(w4, x)
        yc = sk.sk_gemm_w4a8(wc, x)
        torch.cuda.synchronize()
        ref = O.reference(0, buf, n, k, g, x.cpu().numpy())
        assert_y_close(y4.cpu().numpy(), ref)
        assert_y_close(yc.cpu().numpy(), ref)
