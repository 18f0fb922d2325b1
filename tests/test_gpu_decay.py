"""Adagrad Decay (per-period accumulator discount) on the GPU against the
oracle, through the C ABI: rows within the multi-step fp32 bound, each row's
period bit-exact, untouched rows bit-identical.  Cases cover rows finished
inside a reduction chunk, rows spanning chunks of one reduction block
(finished in the block) and rows spanning blocks (finished by the last
block of the span to arrive), sum and mean pooling, and rows wider than 64
lanes."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from recommender_embedding_tables_amd import synth
from tests.helpers import StepBounds, abs_grad_sums

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from recommender_embedding_tables_amd import embtab as eb  # noqa: E402

DEV = torch.device("cuda")
PERIODS = [0, 2, 2, 3, 7]


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def decay_step(tabs, row_periods, offsets, ids, B, pool, grad, lr, eps, rho, period):
    ws, need = tabs.workspace(B, ids.size)
    d_off, d_ids = _t(offsets), _t(ids)
    eb.check(eb.emb_bag_prepare(tabs.handle, d_off, d_ids, B, ids.size, pool, ws, need),
             "prepare")
    eb.check(eb.emb_bag_backward_adagrad_decay_prepared(tabs.handle, B, ids.size, pool, _t(grad),
                                                        lr, eps, rho, period, row_periods, ws,
                                                        need), "decay backward")


def workload(case):
    if case == "one_hot_spans":  # hot rows of table 0 span many chunks
        return synth.workload(2, T=2, B=20000, D=32, rows=[50, 3000]), eb.EMB_POOL_SUM
    if case == "multi_hot_mean":
        w = synth.workload(3, T=2, B=2000, D=64)
        w.rows = np.array([5000, 300])
        return w, eb.EMB_POOL_MEAN
    w = synth.workload(2, T=2, B=3000, D=320, rows=[40, 2000])  # 80 float4 per row
    return w, eb.EMB_POOL_SUM


@pytest.mark.parametrize("case", ["one_hot_spans", "multi_hot_mean", "wide_rows"])
def test_decay_matches_oracle(case):
    w, pool = workload(case)
    rho = 0.6
    tabs = eb.EmbTables(w.rows, w.D, seed=11)
    o = orc.Oracle(w.rows, w.D, seed=11, init_lo=-0.05, init_hi=0.05, accum_init=0.1)
    total = int(np.sum(w.rows))
    row_periods = torch.zeros(total, dtype=torch.int32, device=DEV)
    W0 = tabs.weights.cpu().numpy().copy()
    G0 = tabs.accum.cpu().numpy().copy()
    bounds = StepBounds(total, w.D)
    mean = pool == eb.EMB_POOL_MEAN
    for step, period in enumerate(PERIODS):
        offsets, ids = synth.gen_batch(w, step)
        grad = synth.gen_grad(w, step)
        decay_step(tabs, row_periods, offsets, ids, w.B, pool, grad, w.lr, w.eps, rho, period)
        rows_u, sums = abs_grad_sums(offsets, ids, w.B, o.rows, grad, mean, w.D)
        bounds.step(o, rows_u, sums, w.lr, w.eps,
                    lambda: o.backward_adagrad_decay(offsets, ids, w.B, mean, grad, w.lr, w.eps,
                                                     rho, period))
    torch.cuda.synchronize()
    # periods: bit-exact for every row (untouched rows stay 0)
    np.testing.assert_array_equal(row_periods.cpu().numpy().view(np.uint32),
                                  o.read_periods(np.arange(total)))
    touched = o.touched_rows()
    Wg = tabs.weights[_t(touched)].cpu().numpy()
    Gg = tabs.accum[_t(touched)].cpu().numpy()
    Wr, Gr = o.read_rows(touched)
    # the per-step rule carried over the steps (G' = G*df + g^2 with df <= 1:
    # S_G <= |G| + a^2); exp2f's error in the discount (a few ulp for these
    # exponents) is far inside it
    bounds.check(Wg, Gg, Wr, Gr, touched, f"{len(PERIODS)} decay steps")
    rest = np.setdiff1d(np.arange(total), touched)
    np.testing.assert_array_equal(tabs.weights.cpu().numpy()[rest], W0[rest])
    np.testing.assert_array_equal(tabs.accum.cpu().numpy()[rest], G0[rest])
    assert eb.emb_status_sync(tabs.handle) == (eb.EMB_OK, 0)
    tabs.close()


def test_decay_rho_one_is_bitwise_adagrad():
    # rho = 1: every discount is exp2f(0) = 1, so the rows equal those of the
    # plain prepared backward bit for bit; the periods still advance
    w, pool = workload("one_hot_spans")
    plain = eb.EmbTables(w.rows, w.D, seed=12)
    decay = eb.EmbTables(w.rows, w.D, seed=12)
    total = int(np.sum(w.rows))
    row_periods = torch.zeros(total, dtype=torch.int32, device=DEV)
    for step, period in enumerate(PERIODS[:3]):
        offsets, ids = synth.gen_batch(w, step)
        grad = synth.gen_grad(w, step)
        ws, need = plain.workspace(w.B, ids.size)
        eb.check(eb.emb_bag_prepare(plain.handle, _t(offsets), _t(ids), w.B, ids.size, pool, ws,
                                    need), "prepare")
        eb.check(eb.emb_bag_backward_adagrad_prepared(plain.handle, w.B, ids.size, pool,
                                                      _t(grad), w.lr, w.eps, ws, need),
                 "backward")
        decay_step(decay, row_periods, offsets, ids, w.B, pool, grad, w.lr, w.eps, 1.0, period)
    torch.cuda.synchronize()
    assert torch.equal(plain.weights, decay.weights)
    assert torch.equal(plain.accum, decay.accum)
    assert int(row_periods.max()) == PERIODS[2]
    plain.close()
    decay.close()
