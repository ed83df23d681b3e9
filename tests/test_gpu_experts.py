"""GPU parity of the expert-bank GEMM (flattened E * N rows, one launch over a
per-call expert list) against the oracle and against the plain GEMM run on
each expert's rows alone."""

import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

import gemm_sk_repack_amd as sk  # noqa: E402

from test_gpu_parity import assert_y_close  # noqa: E402


def expert_rows(buf, fmt, n, k, g, e, rows):
    """The canonical bytes of rows [e * rows, (e + 1) * rows) of a bank as a weight of its own."""
    bits = 6 if fmt == 2 else 4
    cb = k * bits // 8
    codes = buf[: n * cb].reshape(n, cb)[e * rows:(e + 1) * rows]
    scales = buf[n * cb:].reshape(n, (k // g) * 4)[e * rows:(e + 1) * rows]
    return np.concatenate([codes.ravel(), scales.ravel()])


@pytest.mark.parametrize("fmt,g", [(0, 32), (2, 64), (0, 128)])
@pytest.mark.parametrize("m", [1, 4, 8])
def test_expert_bank_matches_per_expert_gemm(fmt, g, m):
    E, rows, k = 6, 256, 2048
    n = E * rows
    _, _, buf = S.make_weight(fmt, n, k, g, 1200 + fmt, 1201 + fmt)
    bank = sk.QuantWeight(torch.from_numpy(buf.copy()).cuda(), n, k, g, fmt)
    sk.sk_repack_w4a8(bank)
    experts = [4, 1, 4, 0, 5]
    h = S.activations(1210 + m, m, k)
    x = torch.from_numpy(h).cuda()
    y = sk.sk_gemm_experts(bank, rows, experts, x)
    torch.cuda.synchronize()
    assert y.shape == (m, len(experts) * rows)
    y = y.cpu().numpy()
    for i, e in enumerate(experts):
        sub = expert_rows(buf, fmt, n, k, g, e, rows)
        ref = O.reference(fmt, sub, rows, k, g, h)
        assert_y_close(y[:, i * rows:(i + 1) * rows], ref)
        w = sk.QuantWeight(torch.from_numpy(sub.copy()).cuda(), rows, k, g, fmt)
        sk.sk_repack_w4a8(w)
        y1 = (sk.sk_gemm_w6a8 if fmt == 2 else sk.sk_gemm_w4a8)(w, x).cpu().numpy()
        d = np.abs(y1.astype(np.float64) - y[:, i * rows:(i + 1) * rows])
        assert d.max() <= 1e-6 * max(1.0, np.abs(y1).max()), (e, d.max())
    # repeated ids give repeated blocks, bit for bit
    assert np.array_equal(y[:, 0:rows], y[:, 2 * rows:3 * rows])


def test_expert_bank_single_expert_and_long_k():
    E, rows, k, g = 3, 512, 12288, 32
    n = E * rows
    _, _, buf = S.make_weight(0, n, k, g, 1220, 1221)
    bank = sk.QuantWeight(torch.from_numpy(buf.copy()).cuda(), n, k, g, 0)
    sk.sk_repack_w4a8(bank)
    for m in (1, 3, 8):                    # M = 3: one K-slice with 40 activations per thread
        h = S.activations(1222 + m, m, k)
        y = sk.sk_gemm_experts(bank, rows, [2], torch.from_numpy(h).cuda()).cpu().numpy()
        ref = O.reference(0, expert_rows(buf, 0, n, k, g, 2, rows), rows, k, g, h)
        assert_y_close(y, ref)


def test_expert_bank_rejects_bad_lists():
    E, rows, k, g = 4, 128, 1024, 32
    n = E * rows
    _, _, buf = S.make_weight(0, n, k, g, 1230, 1231)
    bank = sk.QuantWeight(torch.from_numpy(buf.copy()).cuda(), n, k, g, 0)
    x = torch.from_numpy(S.activations(1232, 1, k)).cuda()
    with pytest.raises(sk.SkError) as e:
        sk.sk_gemm_experts(bank, rows, [0], x)          # not repacked
    assert e.value.status == sk.SK_ERR_LAYOUT
    sk.sk_repack_w4a8(bank)
    for bad_rows, ids in ((rows, [E]), (rows, [-1]), (100, [0]), (rows * 3, [0]), (rows, [0] * 65)):
        with pytest.raises(sk.SkError) as e:
            sk.sk_gemm_experts(bank, bad_rows, ids, x)
        assert e.value.status == sk.SK_ERR_SHAPE, (bad_rows, ids)
