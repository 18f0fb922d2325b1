"""The pooled lookup fused with the DLRM dot interaction, forward and
backward, on the GPU against the oracle through the C ABI.  Cases cover one
and two 16-row Gram blocks (T + 1 <= 16 and > 16), the largest shapes
(T = 31, D = 256), widths whose float4 count is not a power of two (D = 48,
112), mean pooling of multi-hot bags, empty bags, absent and
out-of-range ids, rows of more than 128 floats taken in two column halves
(one-hot, multi-hot mean, ragged with empty bags), ten seeded random shapes (T from 1 to 31, D a multiple of
16 up to 256, batches from 1 sample), and a training step whose embedding
gradient comes from the interaction backward."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from recommender_embedding_tables_amd import synth
from tests.helpers import Guarded, abs_grad_sums, assert_within, forward_S

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from recommender_embedding_tables_amd import embtab as eb  # noqa: E402

DEV = torch.device("cuda")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def case(name):
    if name == "one_hot_26":
        return synth.workload(2, T=26, B=3000, D=128,
                              rows=synth.log_uniform_rows(26, 2.0, 5.0, 3, 2)), False
    if name == "multi_hot_mean_8":
        w = synth.workload(3, T=8, B=2000, D=64)
        w.rows = np.full(8, 30_000, np.int64)
        return w, True
    if name == "max_31x256":
        return synth.workload(2, T=31, B=500, D=256, rows=np.full(31, 700)), False
    if name == "multi_hot_d48":  # D / 4 = 12: item tables from a quotient by 12
        w = synth.workload(3, T=13, B=600, D=48)
        w.rows = np.full(13, 5_000, np.int64)
        return w, False
    if name == "one_hot_26_d112":  # D / 4 = 28, 12 items per lane, two row blocks
        return synth.workload(2, T=26, B=700, D=112,
                              rows=synth.log_uniform_rows(26, 2.0, 4.0, 3, 2)), False
    if name == "multi_hot_mean_d256":  # two column halves, bags walked once per half
        w = synth.workload(3, T=5, B=400, D=256)
        w.rows = np.array([3000, 50, 7000, 900, 20], np.int64)
        return w, True
    if name == "ragged_d192":  # two halves of 96 columns, empty bags, absent ids
        w = synth.workload(3, T=7, B=300, D=192)
        w.rows = np.array([40, 900, 7, 300, 60, 5000, 2], np.int64)
        return w, False
    if name.startswith("rand"):  # seeded random shape within the supported range
        rng = np.random.default_rng(700 + int(name[4:]))
        T = int(rng.integers(1, 32))
        D = 16 * int(rng.integers(1, 17))
        B = int(rng.choice([1, 2, 63, 65, int(rng.integers(100, 1500))]))
        w = synth.workload(3, T=T, B=B, D=D)
        w.rows = rng.integers(1, 5_000, size=T).astype(np.int64)
        return w, bool(rng.integers(0, 2))
    w = synth.workload(3, T=5, B=700, D=16)  # ragged bags, some empty
    w.rows = np.array([40, 900, 7, 300, 60], np.int64)
    return w, False


def batch_of(w, name):
    if name in ("small_ragged", "ragged_d192"):  # bags of 0..6 ids, a fifth empty, some absent
        offsets, ids, _ = synth.random_small(8, w.T, w.D, w.B, w.rows, max_len=6, empty_frac=0.2)
        ids = ids.copy()
        ids[::7] = eb.EMB_ID_ABSENT
        return offsets, ids
    if name.startswith("rand"):  # even: one id per bag; odd: ragged bags, some empty
        k = int(name[4:])
        if k % 2 == 0:
            rng = np.random.default_rng(800 + k)
            offsets = np.arange(w.T * w.B + 1, dtype=np.int64)
            ids = np.concatenate([rng.integers(0, r, size=w.B) for r in w.rows]).astype(np.int64)
            return offsets, ids
        offsets, ids, _ = synth.random_small(900 + k, w.T, w.D, w.B, w.rows, max_len=5,
                                             empty_frac=0.15)
        return offsets, ids
    return synth.gen_batch(w, 1)


def z_abs(o, w, offsets, ids, dense, mean):
    """|z| bound of every vector: |dense| and c_b * sum |W| ([B, T + 1, D])."""
    pooled = forward_S(offsets, ids, w.B, o.rows, lambda g: o.read_rows(g)[0], mean, w.D)
    return np.concatenate([np.abs(dense)[:, None, :], pooled], axis=1)


@pytest.mark.parametrize("name", ["one_hot_26", "multi_hot_mean_8", "max_31x256",
                                  "small_ragged", "multi_hot_d48", "one_hot_26_d112",
                                  "multi_hot_mean_d256", "ragged_d192"]
                         + [f"rand{k}" for k in range(10)])
def test_interaction_matches_oracle(name):
    w, mean = case(name)
    pool = eb.EMB_POOL_MEAN if mean else eb.EMB_POOL_SUM
    tabs = eb.EmbTables(w.rows, w.D, seed=9)
    o = orc.Oracle(w.rows, w.D, seed=9, init_lo=-0.05, init_hi=0.05, accum_init=0.1)
    offsets, ids = batch_of(w, name)
    rng = np.random.default_rng(4)
    dense = rng.standard_normal((w.B, w.D)).astype(np.float32)
    odim = eb.emb_interact_out_dim(tabs.handle)
    P = (w.T + 1) * w.T // 2
    assert odim == w.D + P
    out_g = Guarded((w.B, odim), torch.float32, DEV)
    out = out_g.t
    d_off, d_ids, d_dense = _t(offsets), _t(ids), _t(dense)
    eb.check(eb.emb_bag_forward_interact(tabs.handle, d_off, d_ids, w.B, ids.size, pool, d_dense,
                                         out), "forward_interact")
    torch.cuda.synchronize()
    out_g.check("interaction output")
    ref, rc = o.interact_forward(offsets, ids, w.B, mean, dense)
    assert rc == 0
    Z = z_abs(o, w, offsets, ids, dense, mean)
    li, lj = np.tril_indices(w.T + 1, -1)
    S = np.concatenate([np.abs(dense), np.einsum("bid,bjd->bij", Z, Z)[:, li, lj]], axis=1)
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got[:, :w.D], dense)
    assert_within(got, ref, S, "interaction")
    # backward
    g = rng.standard_normal((w.B, odim)).astype(np.float32)
    gd_g = Guarded((w.B, w.D), torch.float32, DEV)
    gp_g = Guarded((w.B, w.T, w.D), torch.float32, DEV)
    gd, gp = gd_g.t, gp_g.t
    eb.check(eb.emb_interact_backward(tabs.handle, d_off, d_ids, w.B, ids.size, pool, d_dense,
                                      _t(g), gd, gp), "interact_backward")
    torch.cuda.synchronize()
    gd_g.check("grad dense")
    gp_g.check("grad pooled")
    rgd, rgp, rc = o.interact_backward(offsets, ids, w.B, mean, dense, g)
    assert rc == 0
    Gs = np.zeros((w.B, w.T + 1, w.T + 1))
    Gs[:, li, lj] = np.abs(g[:, w.D:])
    Gs[:, lj, li] = np.abs(g[:, w.D:])
    SdZ = np.einsum("bij,bjd->bid", Gs, Z)
    assert_within(gd.cpu().numpy(), rgd, np.abs(g[:, :w.D]) + SdZ[:, 0], "grad dense")
    assert_within(gp.cpu().numpy(), rgp, SdZ[:, 1:], "grad pooled")
    flags = eb.emb_status_sync(tabs.handle)
    assert flags == (eb.EMB_OK, 0)
    tabs.close()


def test_out_of_range_ids_and_bad_offsets_are_flagged():
    w, _ = case("small_ragged")
    tabs = eb.EmbTables(w.rows, w.D, seed=9)
    o = orc.Oracle(w.rows, w.D, seed=9, init_lo=-0.05, init_hi=0.05, accum_init=0.1)
    offsets, ids = batch_of(w, "small_ragged")
    ids = ids.copy()
    ids[3] = 10 ** 6  # out of range: contributes 0 and flags
    dense = np.ones((w.B, w.D), np.float32)
    out = torch.empty((w.B, eb.emb_interact_out_dim(tabs.handle)), dtype=torch.float32,
                      device=DEV)
    eb.check(eb.emb_bag_forward_interact(tabs.handle, _t(offsets), _t(ids), w.B, ids.size,
                                         eb.EMB_POOL_SUM, _t(dense), out), "forward_interact")
    ref, _ = o.interact_forward(offsets, ids, w.B, False, dense)
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=1e-5, atol=1e-5)
    assert eb.emb_status_sync(tabs.handle)[0] == eb.EMB_ERR_OUT_OF_RANGE
    bad = offsets.copy()
    bad[5] = bad[6] + 3  # decreasing: those bags count as empty, the call flags
    eb.check(eb.emb_bag_forward_interact(tabs.handle, _t(bad), _t(ids), w.B, ids.size,
                                         eb.EMB_POOL_SUM, _t(dense), out), "forward_interact")
    assert eb.emb_status_sync(tabs.handle)[0] == eb.EMB_ERR_BAD_OFFSETS
    tabs.close()


def test_training_step_through_the_interaction():
    # forward (fused), interaction backward, then the embedding backward with
    # the pooled gradient: rows match the oracle's chain
    w, _ = case("one_hot_26")
    tabs = eb.EmbTables(w.rows, w.D, seed=10)
    o = orc.Oracle(w.rows, w.D, seed=10, init_lo=-0.05, init_hi=0.05, accum_init=0.1)
    offsets, ids = batch_of(w, "one_hot_26")
    rng = np.random.default_rng(6)
    dense = rng.standard_normal((w.B, w.D)).astype(np.float32)
    g = (rng.standard_normal((w.B, eb.emb_interact_out_dim(tabs.handle))) * 0.1).astype(np.float32)
    gd = torch.empty((w.B, w.D), dtype=torch.float32, device=DEV)
    gp = torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=DEV)
    d_off, d_ids = _t(offsets), _t(ids)
    eb.check(eb.emb_interact_backward(tabs.handle, d_off, d_ids, w.B, ids.size, eb.EMB_POOL_SUM,
                                      _t(dense), _t(g), gd, gp), "interact_backward")
    ws, need = tabs.workspace(w.B, ids.size)
    eb.check(eb.emb_bag_backward_adagrad(tabs.handle, d_off, d_ids, w.B, ids.size,
                                         eb.EMB_POOL_SUM, gp, w.lr, w.eps, ws, need), "backward")
    # the pooled gradient the kernel produced is within its bound of the
    # oracle's (the cases above check that); the oracle's step takes the same
    # pooled gradient, so the one-step rule applies to the rows
    _, rgp, _ = o.interact_backward(offsets, ids, w.B, False, dense, g)
    hgp = gp.cpu().numpy()
    li, lj = np.tril_indices(w.T + 1, -1)
    Gs = np.zeros((w.B, w.T + 1, w.T + 1))
    Gs[:, li, lj] = np.abs(g[:, w.D:])
    Gs[:, lj, li] = np.abs(g[:, w.D:])
    Z = z_abs(o, w, offsets, ids, dense, False)
    assert_within(hgp, rgp, np.einsum("bij,bjd->bid", Gs, Z)[:, 1:], "pooled gradient")
    assert o.backward_adagrad(offsets, ids, w.B, False, hgp, w.lr, w.eps) == 0
    uniq, gsum = abs_grad_sums(offsets, ids, w.B, o.rows, hgp, False, w.D)
    Wr, Gr = o.read_rows(uniq)
    SG = np.abs(Gr).astype(np.float64) + gsum ** 2
    SW = np.abs(Wr) + w.lr + w.lr * gsum / (np.sqrt(Gr.astype(np.float64)) + w.eps)
    assert_within(tabs.accum[_t(uniq)].cpu().numpy(), Gr, SG, "accumulator")
    assert_within(tabs.weights[_t(uniq)].cpu().numpy(), Wr, SW, "weights")
    assert eb.emb_status_sync(tabs.handle) == (eb.EMB_OK, 0)
    tabs.close()


def test_interaction_all_bags_empty():
    # nnz = 0: every pooled vector is zero, so the pairs are all zero and the
    # dense slot is copied; the backward gives grad_dense = grad_out's slot
    T, D, B = 5, 32, 300
    rows = np.full(T, 50, np.int64)
    tabs = eb.EmbTables(rows, D, seed=2)
    offsets = np.zeros(T * B + 1, np.int64)
    ids = np.zeros(1, np.int64)
    dense = np.random.default_rng(1).standard_normal((B, D)).astype(np.float32)
    odim = eb.emb_interact_out_dim(tabs.handle)
    out = torch.full((B, odim), 7.0, dtype=torch.float32, device=DEV)
    eb.check(eb.emb_bag_forward_interact(tabs.handle, _t(offsets), _t(ids), B, 0, eb.EMB_POOL_MEAN,
                                         _t(dense), out), "forward_interact")
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got[:, :D], dense)
    np.testing.assert_array_equal(got[:, D:], 0.0)
    g = np.random.default_rng(2).standard_normal((B, odim)).astype(np.float32)
    gd = torch.empty((B, D), dtype=torch.float32, device=DEV)
    gp = torch.empty((B, T, D), dtype=torch.float32, device=DEV)
    eb.check(eb.emb_interact_backward(tabs.handle, _t(offsets), _t(ids), B, 0, eb.EMB_POOL_MEAN,
                                      _t(dense), _t(g), gd, gp), "interact_backward")
    np.testing.assert_array_equal(gd.cpu().numpy(), g[:, :D])  # dz_0 = sum_j g_0j z_j = 0
    # dz_{t+1} = g_{t+1,0} z_0 (the only nonzero vector)
    li, lj = np.tril_indices(T + 1, -1)
    G = np.zeros((B, T + 1, T + 1), np.float64)
    G[:, li, lj] = g[:, D:]
    G[:, lj, li] = g[:, D:]
    ref = G[:, 1:, 0:1] * dense[:, None, :].astype(np.float64)
    np.testing.assert_allclose(gp.cpu().numpy(), ref, rtol=1e-6, atol=1e-7)
    assert eb.emb_status_sync(tabs.handle) == (eb.EMB_OK, 0)
    tabs.close()
