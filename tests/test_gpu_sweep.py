"""Seeded random configurations through the whole prepared path on the GPU,
against the oracle, through the C ABI: the key build, sort and unique of the
prepare, the prepared forward (its one-hot and pooled branches), the forward
that writes the int8 payload, the prepared backward with Adagrad, the one
that reads the int8 gradient payload, and the forward without a workspace.

The hashed sweep runs three calls per configuration: find-or-insert (ids
and the key-to-row map bit for bit), then the prepared step on the ids, with
the per-step rule carried over the steps.

Each configuration draws the table count, the row width (one lane per row up
to several float4 per lane, widths whose float4 count is not a power of two),
the batch size, the bag shape (one id per bag; as many ids as bags without
being one-hot; Poisson bags with empty ones), the pooling, absent ids and
out-of-range ids.  Outputs are compared element by element with the oracle:
copies and integers bit for bit, sums within |err| <= 1e-5 * S + 1e-6, and
every buffer sits between guard bands."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from recommender_embedding_tables_amd import synth
from tests.helpers import REL, Guarded, StepBounds, abs_grad_sums, assert_within, forward_S

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - the marker keeps these off CPU runs
    pytest.skip("needs a GPU", allow_module_level=True)

from recommender_embedding_tables_amd import embtab as eb  # noqa: E402

DEV = torch.device("cuda")
LR, EPS = 0.02, 1e-8


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _config(seed):
    rng = np.random.default_rng(5000 + seed)
    T = int(rng.integers(1, 7))
    D = [4, 8, 12, 20, 36, 60, 64, 100, 128, 132, 256, 260, 516][seed % 13]
    B = int(rng.integers(1000, 8000)) if seed % 2 == 0 else int(rng.choice([1, 3, 64, 257, 4099]))
    kind = ["one_hot", "as_many_as_bags", "poisson"][seed % 3]
    mean = bool(rng.integers(0, 2))
    rows = rng.integers(1, 40_000, size=T).astype(np.int64)
    if kind == "one_hot":
        lens = np.ones(T * B, np.int64)
    elif kind == "as_many_as_bags":
        lens = np.ones(T * B, np.int64)
        k = np.arange(0, T * B - 1, 5)
        lens[k], lens[k + 1] = 2, 0  # nnz = B * T, but not one id per bag
    else:
        lens = rng.poisson(float(rng.uniform(0.5, 12.0)), size=T * B).astype(np.int64)
        lens[rng.random(T * B) < 0.1] = 0
    offsets = synth.offsets_from_lengths(lens)
    ids = np.empty(int(offsets[-1]), np.int64)
    for t in range(T):
        a, b = int(offsets[t * B]), int(offsets[(t + 1) * B])
        ids[a:b] = synth.zipf_ranks(rng, int(rows[t]), float(rng.uniform(0.6, 1.4)), b - a)
    absent = seed % 4 == 1
    oor = seed % 4 == 3
    if ids.size and absent:
        ids[rng.random(ids.size) < 0.05] = eb.EMB_ID_ABSENT
    if ids.size and oor:
        ids[rng.random(ids.size) < 0.03] = -7
        ids[-1] = -7
    grad = rng.standard_normal((B, T, D)).astype(np.float32)
    return dict(T=T, D=D, B=B, kind=kind, mean=mean, rows=rows, offsets=offsets, ids=ids,
                grad=grad, oor=oor and ids.size > 0 and bool(np.any(ids == -7)))


@pytest.mark.parametrize("seed", range(16))
def test_prepared_path_random_config(seed):
    c = _config(seed)
    T, D, B, mean = c["T"], c["D"], c["B"], c["mean"]
    offsets, ids, grad = c["offsets"], c["ids"], c["grad"]
    print(f"seed {seed}: T={T} D={D} B={B} nnz={ids.size} {c['kind']} mean={mean}", flush=True)
    nb, nnz = B * T, ids.size
    pool = eb.EMB_POOL_MEAN if mean else eb.EMB_POOL_SUM
    a = eb.EmbTables(c["rows"], D, seed=seed)    # fp32 gradient
    b = eb.EmbTables(c["rows"], D, seed=seed)    # int8 gradient payload
    o = orc.Oracle(c["rows"], D, seed=seed, init_lo=-0.05, init_hi=0.05, accum_init=0.1)
    d_off, d_ids = _t(offsets), _t(ids)

    # forward without a workspace
    outp = Guarded((B, T, D), torch.float32, DEV)
    eb.check(eb.emb_bag_forward(a.handle, d_off, d_ids, B, nnz, pool, outp.t), "forward")

    # prepare, prepared forward, and the forward that writes the int8 payload
    need = eb.emb_workspace_bytes(a.handle, B, nnz)
    wsa = Guarded(None, torch.uint8, DEV, nbytes=need)
    wsb = Guarded(None, torch.uint8, DEV, nbytes=need)
    eb.check(eb.emb_bag_prepare(a.handle, d_off, d_ids, B, nnz, pool, wsa.t, need), "prepare a")
    eb.check(eb.emb_bag_prepare(b.handle, d_off, d_ids, B, nnz, pool, wsb.t, need), "prepare b")
    out = Guarded((B, T, D), torch.float32, DEV)
    out.t.fill_(float("nan"))
    eb.check(eb.emb_bag_forward_prepared(a.handle, d_off, d_ids, B, nnz, pool, out.t, wsa.t,
                                         need), "forward_prepared")
    cg = Guarded((nb, D), torch.int8, DEV)
    sg = Guarded((nb,), torch.float32, DEV)
    eb.check(eb.emb_bag_forward_prepared_int8(a.handle, d_off, d_ids, B, nnz, pool, cg.t, sg.t,
                                              wsa.t, need), "forward_prepared_int8")
    c2 = torch.empty((nb, D), dtype=torch.int8, device=DEV)
    s2 = torch.empty(nb, dtype=torch.float32, device=DEV)
    if nb:
        eb.check(eb.emb_quantize_rows_int8(out.t, nb, D, c2, s2), "quantize")
    torch.cuda.synchronize()
    for g, what in ((outp, "forward output"), (out, "prepared forward output"),
                    (cg, "payload codes"), (sg, "payload scales"), (wsa, "workspace a"),
                    (wsb, "workspace b")):
        g.check(what)

    ref, fl = o.forward(offsets, ids, B, mean)
    assert fl == (1 if c["oor"] else 0)
    got = out.t.cpu().numpy()
    if nnz == 0 or np.diff(offsets).max() <= 1:  # copies of one row, or zeros
        np.testing.assert_array_equal(got, ref)
        np.testing.assert_array_equal(outp.t.cpu().numpy(), ref)
    else:
        S = forward_S(offsets, ids, B, o.rows, lambda r: o.read_rows(r)[0], mean, D)
        assert_within(got, ref, S, "prepared forward")
        assert_within(outp.t.cpu().numpy(), ref, S, "forward")
    # the fused payload equals the stand-alone quantization of the same rows
    np.testing.assert_array_equal(cg.t.cpu().numpy(), c2.cpu().numpy())
    np.testing.assert_array_equal(sg.t.cpu().numpy(), s2.cpu().numpy())

    # backward: fp32 gradient (already on the payload's grid) on a, payload on b
    codes, scales = orc.quantize_rows_int8(grad.reshape(nb, D))
    gdq = orc.dequantize_rows_int8(codes, scales).reshape(B, T, D)
    gc = Guarded((nb, D), torch.int8, DEV)
    gs = Guarded((nb,), torch.float32, DEV)
    gc.t.copy_(torch.from_numpy(codes))
    gs.t.copy_(torch.from_numpy(scales))
    eb.check(eb.emb_bag_backward_adagrad_prepared(a.handle, B, nnz, pool, _t(gdq), LR, EPS,
                                                  wsa.t, need), "backward_prepared")
    eb.check(eb.emb_bag_backward_adagrad_prepared_int8(b.handle, B, nnz, pool, gc.t, gs.t, LR,
                                                       EPS, wsb.t, need), "backward_int8")
    torch.cuda.synchronize()
    for g, what in ((gc, "gradient codes"), (gs, "gradient scales"), (wsa, "workspace a"),
                    (wsb, "workspace b")):
        g.check(what + " after the backward")
    assert torch.equal(a.weights, b.weights) and torch.equal(a.accum, b.accum)

    assert o.backward_adagrad(offsets, ids, B, mean, gdq, LR, EPS) == (1 if c["oor"] else 0)
    uniq, gsum = abs_grad_sums(offsets, ids, B, o.rows, gdq, mean, D)
    if uniq.size:
        Wr, Gr = o.read_rows(uniq)
        SG = np.abs(Gr).astype(np.float64) + gsum ** 2
        SW = np.abs(Wr) + LR + LR * gsum / (np.sqrt(Gr.astype(np.float64)) + EPS)
        assert_within(a.accum[_t(uniq)].cpu().numpy(), Gr, SG, "accumulator")
        assert_within(a.weights[_t(uniq)].cpu().numpy(), Wr, SW, "weights")
    # rows the batch does not touch are left as they were, bit for bit
    rest = np.setdiff1d(np.arange(0, int(c["rows"].sum()), 7), uniq)
    if rest.size:
        Wr, Gr = o.read_rows(rest)
        np.testing.assert_array_equal(a.weights[_t(rest)].cpu().numpy(), Wr)
        np.testing.assert_array_equal(a.accum[_t(rest)].cpu().numpy(), Gr)

    torch.cuda.synchronize()
    # out-of-range ids are skipped and reported (the report clears on reading)
    want = (eb.EMB_ERR_OUT_OF_RANGE, eb.EMB_FLAG_OUT_OF_RANGE) if c["oor"] else (eb.EMB_OK, 0)
    for tabs in (a, b):
        assert eb.emb_status_sync(tabs.handle) == want
        assert eb.emb_status_sync(tabs.handle) == (eb.EMB_OK, 0)


@pytest.mark.parametrize("seed", range(8))
def test_hashed_prepared_path_random_config(seed):
    rng = np.random.default_rng(6000 + seed)
    T = int(rng.integers(1, 5))
    D = [4, 12, 36, 64, 100, 128, 260, 516][seed]
    cap = 1 << int(rng.integers(10, 15))
    rows = np.full(T, int(0.625 * cap), np.int64)
    B = int(rng.choice([1, 5, 200, int(rng.integers(500, 3000))]))
    mean = bool(rng.integers(0, 2))
    kind = ["one_hot", "poisson", "as_many_as_bags"][seed % 3]
    # each table's keys come from a universe no larger than its rows: no call is full
    univ = [rng.integers(1, 2 ** 63, size=int(rng.integers(1, rows[0] + 1)), dtype=np.uint64)
            for _ in range(T)]
    print(f"seed {seed}: T={T} D={D} cap={cap} B={B} {kind} mean={mean} "
          f"universe={[u.size for u in univ]}", flush=True)
    pool = eb.EMB_POOL_MEAN if mean else eb.EMB_POOL_SUM
    kw = dict(seed=seed, init_lo=-0.05, init_hi=0.05, init_std=0.01, accum_init=0.1)
    tabs = eb.EmbTables(rows, D, hashed=True, hash_capacity=cap, max_load=0.625, **kw)
    o = orc.Oracle(rows, D, hashed=True, **kw)
    bounds = StepBounds(int(rows.sum()), D)
    row_off = np.concatenate([[0], np.cumsum(rows)])
    live = lambda: np.concatenate([np.arange(o.n_live(t)) + row_off[t]  # noqa: E731
                                   for t in range(T)])
    live_before = live()
    for call in range(3):
        if kind == "one_hot":
            lens = np.ones(T * B, np.int64)
        elif kind == "as_many_as_bags":
            lens = np.ones(T * B, np.int64)
            k = np.arange(call % 2, T * B - 1, 4)
            lens[k], lens[k + 1] = 2, 0
        else:
            lens = rng.poisson(3.0, size=T * B).astype(np.int64)
        offsets = synth.offsets_from_lengths(lens)
        nnz = int(offsets[-1])
        keys = np.empty(nnz, np.uint64)
        for t in range(T):
            a, b = int(offsets[t * B]), int(offsets[(t + 1) * B])
            keys[a:b] = univ[t][synth.zipf_ranks(rng, univ[t].size, 1.1, b - a)]
        d_off = _t(offsets)
        need = eb.emb_workspace_bytes(tabs.handle, B, nnz)
        ws = Guarded(None, torch.uint8, DEV, nbytes=need)
        idg = Guarded((nnz,), torch.int64, DEV)
        eb.check(eb.emb_hash_find_or_insert(tabs.handle, d_off, _t(keys.view(np.int64)), B, nnz,
                                            idg.t, ws.t, need), "find_or_insert")
        torch.cuda.synchronize()
        ref_ids, fl = o.find_or_insert(offsets, keys, B)
        assert fl == 0
        np.testing.assert_array_equal(idg.t.cpu().numpy(), ref_ids)
        live_now = live()
        bounds.assigned(o, np.setdiff1d(live_now, live_before))
        live_before = live_now

        grad = rng.standard_normal((B, T, D)).astype(np.float32)
        out = Guarded((B, T, D), torch.float32, DEV)
        eb.check(eb.emb_bag_prepare(tabs.handle, d_off, idg.t, B, nnz, pool, ws.t, need),
                 "prepare")
        eb.check(eb.emb_bag_forward_prepared(tabs.handle, d_off, idg.t, B, nnz, pool, out.t,
                                             ws.t, need), "forward_prepared")
        torch.cuda.synchronize()
        got = out.t.cpu().numpy()
        eb.check(eb.emb_bag_backward_adagrad_prepared(tabs.handle, B, nnz, pool, _t(grad), LR,
                                                      EPS, ws.t, need), "backward_prepared")
        torch.cuda.synchronize()
        for g, what in ((ws, "workspace"), (idg, "ids"), (out, "forward output")):
            g.check(f"{what}, call {call}")

        ref, _ = o.forward(offsets, ref_ids, B, mean)
        S = forward_S(offsets, ref_ids, B, o.rows, lambda r: np.abs(o.read_rows(r)[0]), mean, D)
        S = S + forward_S(offsets, ref_ids, B, o.rows, bounds.weight_bound, mean, D) / REL
        assert_within(got, ref, S, f"forward, call {call}")
        uniq, gsum = abs_grad_sums(offsets, ref_ids, B, o.rows, grad, mean, D)
        assert bounds.step(o, uniq, gsum, LR, EPS, lambda: o.backward_adagrad(
            offsets, ref_ids, B, mean, grad, LR, EPS)) == 0
        if uniq.size:
            Wr, Gr = o.read_rows(uniq)
            bounds.check(tabs.weights[_t(uniq)].cpu().numpy(), tabs.accum[_t(uniq)].cpu().numpy(),
                         Wr, Gr, uniq, f"rows, call {call}")
    # the key -> row map, bit for bit
    st, n_live = eb.emb_hash_n_live(tabs.handle, T)
    assert st == eb.EMB_OK
    for t in range(T):
        assert n_live[t] == o.n_live(t)
        kor = torch.empty(int(rows[t]), dtype=torch.int64, device=DEV)
        eb.check(eb.emb_hash_export(tabs.handle, t, kor), "export")
        k_t, r_t = o.export(t)
        want = np.empty(n_live[t], np.uint64)
        want[r_t] = k_t
        torch.cuda.synchronize()
        np.testing.assert_array_equal(kor[:n_live[t]].cpu().numpy().view(np.uint64), want)
    assert eb.emb_status_sync(tabs.handle) == (eb.EMB_OK, 0)
    tabs.close()
