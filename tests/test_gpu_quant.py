"""The int8 exchange payload on the GPU against the oracle, through the C ABI:
codes and scales bit for bit (both sides decide each code in fp32 with the
same operations), dequantized rows bit for bit.  Shapes cover one lane per
row (D = 4), sub-groups with idle lanes (D = 12, 20), the pooled rows of the
26-table workload (D = 128) at their full count (65536 x 26 rows), several
float4 per lane (D = 1024), zero rows, rows with ties, and guard bands."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from tests.helpers import Guarded

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from recommender_embedding_tables_amd import embtab as eb  # noqa: E402

DEV = torch.device("cuda")


def _rows(rows, D, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, D)) * np.exp(rng.uniform(-6, 6, (rows, 1)))).astype(np.float32)
    if rows > 3:
        x[1] = 0.0
        # amax 127 gives inv = 1: halves are ties, which go to even
        x[2] = (np.arange(D) % 9 - 4).astype(np.float32) + np.float32(0.5)
        x[2, 0] = 127.0
    return x


def _gpu(x):
    rows, D = x.shape
    xd = torch.from_numpy(x).to(DEV)
    cg = Guarded((rows, D), torch.int8, DEV)
    sg = Guarded((rows,), torch.float32, DEV)
    eb.check(eb.emb_quantize_rows_int8(xd, rows, D, cg.t, sg.t), "quantize")
    yg = Guarded((rows, D), torch.float32, DEV)
    eb.check(eb.emb_dequantize_rows_int8(cg.t, sg.t, rows, D, yg.t), "dequantize")
    torch.cuda.synchronize()
    cg.check("codes")
    sg.check("scales")
    yg.check("dequantized")
    return cg.t.cpu().numpy(), sg.t.cpu().numpy(), yg.t.cpu().numpy()


@pytest.mark.parametrize("rows,D", [(1, 4), (37, 12), (300, 20), (1000, 128), (333, 256),
                                    (64, 1024), (5, 16)])
def test_int8_payload_matches_oracle(rows, D):
    x = _rows(rows, D, rows * 7 + D)
    codes, scales, y = _gpu(x)
    rc, rs = orc.quantize_rows_int8(x)
    np.testing.assert_array_equal(codes, rc)
    np.testing.assert_array_equal(scales.view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(y.view(np.uint32),
                                  orc.dequantize_rows_int8(rc, rs).view(np.uint32))


def test_int8_payload_full_pooled_shape():
    # the pooled output of 26 tables at B = 65536, D = 128: 1.7M rows
    rows, D = 65536 * 26, 128
    x = _rows(rows, D, 11)
    codes, scales, y = _gpu(x)
    rc, rs = orc.quantize_rows_int8(x)
    np.testing.assert_array_equal(codes, rc)
    np.testing.assert_array_equal(scales, rs)
    np.testing.assert_array_equal(y, orc.dequantize_rows_int8(rc, rs))


# ------------------------------------------------ forward writing the payload

from recommender_embedding_tables_amd import synth  # noqa: E402
from tests.helpers import forward_S  # noqa: E402


def _workload(name):
    if name == "one_hot":
        return synth.workload(2, T=26, B=2000, D=128,
                              rows=synth.log_uniform_rows(26, 2.0, 5.0, 3, 2))
    w = synth.workload(3, T=6, B=500, D=64)
    w.rows = np.full(6, 20_000, np.int64)
    w.pool_mean = name == "multi_hot_mean"
    return w


@pytest.mark.parametrize("name", ["one_hot", "multi_hot_sum", "multi_hot_mean"])
def test_forward_prepared_int8(name):
    w = _workload(name)
    tabs = eb.EmbTables(w.rows, w.D, seed=5)
    o = orc.Oracle(w.rows, w.D, seed=5, init_lo=-0.05, init_hi=0.05, accum_init=0.1)
    offsets, ids = synth.gen_batch(w, 0)
    d_off, d_ids = torch.from_numpy(offsets).to(DEV), torch.from_numpy(ids).to(DEV)
    pool = eb.EMB_POOL_MEAN if w.pool_mean else eb.EMB_POOL_SUM
    nb = w.B * w.T
    ws, need = tabs.workspace(w.B, ids.size)
    eb.check(eb.emb_bag_prepare(tabs.handle, d_off, d_ids, w.B, ids.size, pool, ws, need),
             "prepare")
    cg = Guarded((nb, w.D), torch.int8, DEV)
    sg = Guarded((nb,), torch.float32, DEV)
    eb.check(eb.emb_bag_forward_prepared_int8(tabs.handle, d_off, d_ids, w.B, ids.size, pool,
                                              cg.t, sg.t, ws, need), "forward_prepared_int8")
    # the same launch writing fp32 rows, quantized by the stand-alone kernel:
    # the fused payload equals it bit for bit
    out = torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=DEV)
    eb.check(eb.emb_bag_forward_prepared(tabs.handle, d_off, d_ids, w.B, ids.size, pool, out,
                                         ws, need), "forward_prepared")
    c2 = torch.empty((nb, w.D), dtype=torch.int8, device=DEV)
    s2 = torch.empty(nb, dtype=torch.float32, device=DEV)
    eb.check(eb.emb_quantize_rows_int8(out, nb, w.D, c2, s2), "quantize")
    torch.cuda.synchronize()
    cg.check("codes")
    sg.check("scales")
    codes, scales = cg.t.cpu().numpy(), sg.t.cpu().numpy()
    np.testing.assert_array_equal(codes, c2.cpu().numpy())
    np.testing.assert_array_equal(scales, s2.cpu().numpy())
    assert eb.emb_status_sync(tabs.handle) == (eb.EMB_OK, 0)
    # against the oracle: its pooled rows quantized by its own payload function
    ref, _ = o.forward(offsets, ids, w.B, w.pool_mean)
    rc, rs = orc.quantize_rows_int8(ref.reshape(nb, w.D))
    if name == "one_hot":  # a one-hot row is a copy: exact
        np.testing.assert_array_equal(codes, rc)
        np.testing.assert_array_equal(scales, rs)
        return
    # multi-hot: the fp32 sum may differ from the rounded exact sum within the
    # pooled tolerance, which can move a code by one and the scale slightly
    S = forward_S(offsets, ids, w.B, o.rows, lambda g: o.read_rows(g)[0], w.pool_mean,
                  w.D).reshape(nb, w.D)
    tol = 1e-5 * S + 1e-6
    assert np.all(np.abs(codes.astype(np.int32) - rc.astype(np.int32)) <= 1)
    assert np.all(np.abs(scales - rs) <= tol.max(axis=1) / 127 + 2 ** -22 * rs)
    deq = codes.astype(np.float64) * scales[:, None]
    assert np.all(np.abs(deq - ref.reshape(nb, w.D)) <=
                  0.5 * scales[:, None] * (1 + 1e-5) + tol + 2 ** -22 * np.abs(deq))


# ------------------------------------ backward reading the received payload

from tests.helpers import StepBounds, abs_grad_sums  # noqa: E402


@pytest.mark.parametrize("name", ["one_hot", "multi_hot_sum", "multi_hot_mean"])
def test_backward_prepared_int8(name):
    w = _workload(name)
    a = eb.EmbTables(w.rows, w.D, seed=6)
    b = eb.EmbTables(w.rows, w.D, seed=6)
    o = orc.Oracle(w.rows, w.D, seed=6, init_lo=-0.05, init_hi=0.05, accum_init=0.1)
    offsets, ids = synth.gen_batch(w, 1)
    d_off, d_ids = torch.from_numpy(offsets).to(DEV), torch.from_numpy(ids).to(DEV)
    pool = eb.EMB_POOL_MEAN if w.pool_mean else eb.EMB_POOL_SUM
    nb = w.B * w.T
    grad = np.random.default_rng(3).standard_normal((nb, w.D)).astype(np.float32)
    codes, scales = orc.quantize_rows_int8(grad)
    gdq = orc.dequantize_rows_int8(codes, scales).reshape(w.B, w.T, w.D)
    lr, eps = 0.01, 1e-8
    for tabs in (a, b):
        ws, need = tabs.workspace(w.B, ids.size)
        eb.check(eb.emb_bag_prepare(tabs.handle, d_off, d_ids, w.B, ids.size, pool, ws, need),
                 "prepare")
        if tabs is a:
            cg = Guarded((nb, w.D), torch.int8, DEV)
            sg = Guarded((nb,), torch.float32, DEV)
            cg.t.copy_(torch.from_numpy(codes))
            sg.t.copy_(torch.from_numpy(scales))
            eb.check(eb.emb_bag_backward_adagrad_prepared_int8(
                a.handle, w.B, ids.size, pool, cg.t, sg.t, lr, eps, ws, need), "backward_int8")
        else:
            eb.check(eb.emb_bag_backward_adagrad_prepared(
                b.handle, w.B, ids.size, pool, torch.from_numpy(gdq).to(DEV), lr, eps, ws, need),
                "backward")
        torch.cuda.synchronize()
    cg.check("grad codes")
    sg.check("grad scales")
    # the payload read in place of its dequantized rows: the same tables bit for bit
    assert torch.equal(a.weights, b.weights) and torch.equal(a.accum, b.accum)
    assert eb.emb_status_sync(a.handle) == (eb.EMB_OK, 0)
    # and the oracle's step on the dequantized gradient, within the per-step rule
    bounds = StepBounds(sum(w.rows), w.D)
    uniq, gsum = abs_grad_sums(offsets, ids, w.B, o.rows, gdq, w.pool_mean, w.D)
    assert bounds.step(o, uniq, gsum, lr, eps, lambda: o.backward_adagrad(
        offsets, ids, w.B, w.pool_mean, gdq, lr, eps)) == 0
    Wr, Gr = o.read_rows(uniq)
    bounds.check(a.weights[torch.from_numpy(uniq).to(DEV)].cpu().numpy(),
                 a.accum[torch.from_numpy(uniq).to(DEV)].cpu().numpy(), Wr, Gr, uniq, "rows")
