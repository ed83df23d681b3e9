"""GPU parity of the expert-bank GEMM (flattened E * N rows, one launch over a
device list of expert ids) against the oracle and against the plain GEMM run
on each expert's rows alone."""

import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

import gemm_sk_repack_amd as sk  # noqa: E402

from test_gpu_parity import assert_y_close  # noqa: E402


def ids(lst):
    return torch.tensor(lst, dtype=torch.int32, device="cuda")


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
    y = sk.sk_gemm_experts(bank, rows, ids(experts), x)
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
        y = sk.sk_gemm_experts(bank, rows, ids([2]), torch.from_numpy(h).cuda()).cpu().numpy()
        ref = O.reference(0, expert_rows(buf, 0, n, k, g, 2, rows), rows, k, g, h)
        assert_y_close(y, ref)


def test_expert_bank_rejects_bad_shapes():
    E, rows, k, g = 4, 128, 1024, 32
    n = E * rows
    _, _, buf = S.make_weight(0, n, k, g, 1230, 1231)
    bank = sk.QuantWeight(torch.from_numpy(buf.copy()).cuda(), n, k, g, 0)
    x = torch.from_numpy(S.activations(1232, 1, k)).cuda()
    with pytest.raises(sk.SkError) as e:
        sk.sk_gemm_experts(bank, rows, ids([0]), x)          # not repacked
    assert e.value.status == sk.SK_ERR_LAYOUT
    sk.sk_repack_w4a8(bank)
    for bad_rows in (100, rows * 3):
        with pytest.raises(sk.SkError) as e:
            sk.sk_gemm_experts(bank, bad_rows, ids([0]), x)
        assert e.value.status == sk.SK_ERR_SHAPE, bad_rows


@pytest.mark.parametrize("m", [1, 8])
def test_expert_ids_outside_the_bank_give_nan_blocks(m):
    """Ids are read on the device, so an id outside [0, E) cannot be rejected on
    the host: its block of y is NaN and the other blocks are unaffected."""
    E, rows, k, g = 4, 128, 1024, 32
    n = E * rows
    _, _, buf = S.make_weight(0, n, k, g, 1240, 1241)
    bank = sk.QuantWeight(torch.from_numpy(buf.copy()).cuda(), n, k, g, 0)
    sk.sk_repack_w4a8(bank)
    h = S.activations(1242 + m, m, k)
    lst = [1, E, 3, -1, 0, 1 << 20]
    y = sk.sk_gemm_experts(bank, rows, ids(lst), torch.from_numpy(h).cuda()).cpu().numpy()
    for i, e in enumerate(lst):
        blk = y[:, i * rows:(i + 1) * rows]
        if 0 <= e < E:
            assert_y_close(blk, O.reference(0, expert_rows(buf, 0, n, k, g, e, rows), rows, k, g, h))
        else:
            assert np.all(np.isnan(blk)), e


def test_expert_list_changes_between_graph_replays():
    """A captured call reads the device list when it runs: the router's output
    can change between replays without capturing again."""
    E, rows, k, g, m = 8, 256, 2048, 32, 4
    n = E * rows
    _, _, buf = S.make_weight(0, n, k, g, 1250, 1251)
    bank = sk.QuantWeight(torch.from_numpy(buf.copy()).cuda(), n, k, g, 0)
    sk.sk_repack_w4a8(bank)
    h = S.activations(1252, m, k)
    x = torch.from_numpy(h).cuda()
    lst = ids([0, 1, 2])
    y = torch.empty((m, 3 * rows), dtype=torch.float32, device="cuda")
    sk.sk_gemm_experts(bank, rows, lst, x, y=y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sk.sk_gemm_experts(bank, rows, lst, x, y=y)
    rng = np.random.default_rng(1253)
    for rep in range(4):
        chosen = rng.choice(E, 3, replace=rep % 2 == 0).astype(np.int32)
        lst.copy_(torch.from_numpy(chosen))
        graph.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        for i, e in enumerate(chosen):
            ref = O.reference(0, expert_rows(buf, 0, n, k, g, int(e), rows), rows, k, g, h)
            assert_y_close(got[:, i * rows:(i + 1) * rows], ref)
