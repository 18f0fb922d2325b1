"""The dense-table schedule bench.py runs for long bags, against the oracle
through the C ABI: the prepare of batch i+2 on one of two side streams
(alternating), beside the forward and backward of batch i on the main
stream, with three workspaces.  Prepares read only ids, so two of them may
run at once; every result equals the sequential one (pooled outputs and
rows within the per-step rule carried over the steps, untouched rows
bit-identical)."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from recommender_embedding_tables_amd import synth
from tests.helpers import REL, StepBounds, abs_grad_sums, assert_within, forward_S

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from recommender_embedding_tables_amd import embtab as eb  # noqa: E402

DEV = torch.device("cuda")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_dense_two_prepares_in_flight():
    w = synth.workload(3, T=3, B=2500)
    w.rows = np.array([40_000, 300, 7_000])
    steps = 6
    pool = eb.EMB_POOL_MEAN
    tabs = eb.EmbTables(w.rows, w.D, seed=21)
    o = orc.Oracle(w.rows, w.D, seed=21)
    W0 = tabs.weights.cpu().numpy().copy()
    G0 = tabs.accum.cpu().numpy().copy()
    host = [synth.gen_batch(w, b) for b in range(steps)]
    dev = [(_t(off), _t(ids)) for off, ids in host]
    grads = [synth.gen_grad(w, b) for b in range(steps)]
    nnz = max(ids.size for _, ids in host)
    ws0, need = tabs.workspace(w.B, nnz)
    wss = [ws0, torch.empty_like(ws0), torch.empty_like(ws0)]
    outs = [torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=DEV) for _ in range(steps)]
    main = torch.cuda.current_stream()
    sides = [torch.cuda.Stream(), torch.cuda.Stream()]
    prepared = [torch.cuda.Event() for _ in range(steps)]
    trained = [torch.cuda.Event() for _ in range(steps)]

    def prepare(i):
        if i >= steps:
            return
        s = sides[i % 2]
        if i >= 3:
            s.wait_event(trained[i - 3])  # batch i - 3 used this workspace
        d_off, d_ids = dev[i]
        eb.check(eb.emb_bag_prepare(tabs.handle, d_off, d_ids, w.B, d_ids.numel(), pool,
                                    wss[i % 3], need, s), "prepare")
        prepared[i].record(s)

    prepare(0)
    prepare(1)
    for i in range(steps):
        prepare(i + 2)
        main.wait_event(prepared[i])
        d_off, d_ids = dev[i]
        eb.check(eb.emb_bag_forward_prepared(tabs.handle, d_off, d_ids, w.B, d_ids.numel(), pool,
                                             outs[i], wss[i % 3], need, main), "forward")
        eb.check(eb.emb_bag_backward_adagrad_prepared(tabs.handle, w.B, d_ids.numel(), pool,
                                                      _t(grads[i]), w.lr, w.eps, wss[i % 3],
                                                      need, main), "backward")
        trained[i].record(main)
    torch.cuda.synchronize()

    # the oracle replays the steps in order, carrying the per-step rule
    bounds = StepBounds(int(np.sum(w.rows)), w.D)
    for i in range(steps):
        offsets, ids = host[i]
        ref, _ = o.forward(offsets, ids, w.B, True)
        S = forward_S(offsets, ids, w.B, o.rows, lambda r: np.abs(o.read_rows(r)[0]), True, w.D)
        S = S + forward_S(offsets, ids, w.B, o.rows, bounds.weight_bound, True, w.D) / REL
        assert_within(outs[i].cpu().numpy(), ref, S, f"pooled output of step {i}")
        uniq, gsum = abs_grad_sums(offsets, ids, w.B, o.rows, grads[i], True, w.D)
        assert bounds.step(o, uniq, gsum, w.lr, w.eps, lambda: o.backward_adagrad(
            offsets, ids, w.B, True, grads[i], w.lr, w.eps)) == 0
    rows = o.touched_rows()
    Wr, Gr = o.read_rows(rows)
    bounds.check(tabs.weights[_t(rows)].cpu().numpy(), tabs.accum[_t(rows)].cpu().numpy(),
                 Wr, Gr, rows, "rows after the steps")
    rest = np.setdiff1d(np.arange(int(np.sum(w.rows))), rows)
    np.testing.assert_array_equal(tabs.weights.cpu().numpy()[rest], W0[rest])
    np.testing.assert_array_equal(tabs.accum.cpu().numpy()[rest], G0[rest])
    assert eb.emb_status_sync(tabs.handle) == (eb.EMB_OK, 0)
    tabs.close()
