"""Frequency admission on the GPU hash against the oracle, through the C ABI:
ids bit-exact every call (rows, -1, and -2 for keys not admitted yet), the
key<->row map and the new rows' values, full calls, and a training step on
ids that hold absent features."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from recommender_embedding_tables_amd import synth
from tests.helpers import (REL, StepBounds, abs_grad_sums, assert_within, forward_S, key_rows,
                           rows_given_keys)
from tests.test_gpu_parity import _hash_call, _t, check_hash_state, make_pair, status

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from recommender_embedding_tables_amd import embtab as eb  # noqa: E402

DEV = torch.device("cuda")


def counts_for(tabs):
    return torch.zeros(tabs.T * tabs.hash_capacity, dtype=torch.int32, device=DEV)


def admit_call(tabs, counts, offsets, keys, B, N):
    ids = torch.empty(keys.size, dtype=torch.int64, device=DEV)
    ws, need = tabs.workspace(B, keys.size)
    eb.check(eb.emb_hash_find_or_insert_admit(tabs.handle, _t(offsets), _t(keys.view(np.int64)),
                                              B, keys.size, ids, N, counts, ws, need),
             "find_or_insert_admit")
    torch.cuda.synchronize()
    return ids.cpu().numpy()


@pytest.mark.parametrize("N", [2, 4])
def test_admission_matches_oracle_over_calls(N):
    w = synth.workload(5, T=3, B=3000, universe=40_000, hash_capacity=1 << 16)
    w.rows = np.full(3, int(0.625 * (1 << 16)), np.int64)
    tabs, o = make_pair(w.rows, w.D, seed=23, hashed=True, cap=w.hash_capacity)
    counts = counts_for(tabs)
    absent = 0
    for step in range(6):
        offsets, ranks = synth.gen_batch(w, step)
        keys = synth.gen_keys(w, offsets, ranks)
        ids = admit_call(tabs, counts, offsets, keys, w.B, N)
        ref, fl = o.find_or_insert_admit(offsets, keys, w.B, N)
        assert fl == 0
        np.testing.assert_array_equal(ids, ref)
        absent += int((ids == eb.EMB_ID_ABSENT).sum())
        assert status(tabs) == (eb.EMB_OK, 0)
    assert absent > 0
    check_hash_state(tabs, o)


def test_admission_min_count_one_equals_insertion():
    w = synth.workload(5, T=2, B=2000, universe=30_000, hash_capacity=1 << 15)
    w.rows = np.full(2, int(0.625 * (1 << 15)), np.int64)
    plain, _ = make_pair(w.rows, w.D, seed=5, hashed=True, cap=w.hash_capacity)
    admit, _ = make_pair(w.rows, w.D, seed=5, hashed=True, cap=w.hash_capacity)
    for step in range(3):
        offsets, ranks = synth.gen_batch(w, step)
        keys = synth.gen_keys(w, offsets, ranks)
        np.testing.assert_array_equal(_hash_call(plain, offsets, keys, w.B),
                                      admit_call(admit, None, offsets, keys, w.B, 1))
    st, n_live = eb.emb_hash_n_live(admit.handle, admit.T)
    assert st == eb.EMB_OK and eb.emb_hash_n_live(plain.handle, plain.T)[1] == n_live
    for t in range(admit.T):  # rows handed out (the others hold no defined value)
        a = int(np.sum(w.rows[:t]))
        assert torch.equal(plain.weights[a:a + n_live[t]], admit.weights[a:a + n_live[t]])


def test_admission_full_call_admits_nothing_then_admits_at_once():
    rows = np.array([6, 50])
    tabs, o = make_pair(rows, 8, hashed=True, cap=128, seed=3)
    counts = counts_for(tabs)
    N = 2
    off = np.array([0, 5, 7], np.int64)  # B = 1
    k1 = np.array([1, 2, 3, 1, 2, 40, 41], np.uint64)  # 1 and 2 admitted in table 0
    np.testing.assert_array_equal(admit_call(tabs, counts, off, k1, 1, N),
                                  o.find_or_insert_admit(off, k1, 1, N)[0])
    # table 0 would need 2 + 5 > 6 rows: nothing is admitted, counts advance
    off2 = np.array([0, 10, 12], np.int64)
    k2 = np.array([3, 4, 4, 5, 5, 6, 6, 7, 7, 1, 40, 41], np.uint64)
    ids_g = admit_call(tabs, counts, off2, k2, 1, N)
    ids_r, fl = o.find_or_insert_admit(off2, k2, 1, N)
    assert fl == orc.ERR_TABLE_FULL
    np.testing.assert_array_equal(ids_g, ids_r)
    assert status(tabs) == (eb.EMB_ERR_TABLE_FULL, eb.EMB_FLAG_TABLE_FULL)
    # with room (one key each): 4 reached 2 before and is admitted at first sight
    off3 = np.array([0, 2, 3], np.int64)
    k3 = np.array([4, 9, 40], np.uint64)
    np.testing.assert_array_equal(admit_call(tabs, counts, off3, k3, 1, N),
                                  o.find_or_insert_admit(off3, k3, 1, N)[0])
    check_hash_state(tabs, o)


def test_training_on_absent_ids():
    # absent features look up 0 (counted in mean bags), get no update and raise no error
    w = synth.workload(5, T=2, B=1500, universe=20_000, hash_capacity=1 << 15)
    w.rows = np.full(2, int(0.625 * (1 << 15)), np.int64)
    tabs, o = make_pair(w.rows, w.D, seed=8, hashed=True, cap=w.hash_capacity)
    counts = counts_for(tabs)
    # the per-step rule carried over the steps (tests/helpers.py StepBounds);
    # a lookup of a row adds that row's carried weight bound to its term
    bounds = StepBounds(int(np.sum(w.rows)), w.D)
    for step in range(3):
        offsets, ranks = synth.gen_batch(w, step)
        keys = synth.gen_keys(w, offsets, ranks)
        ids = admit_call(tabs, counts, offsets, keys, w.B, 3)
        before = key_rows(o)
        ref, _ = o.find_or_insert_admit(offsets, keys, w.B, 3)
        bounds.assigned(o, rows_given_keys(before, key_rows(o)))
        np.testing.assert_array_equal(ids, ref)
        assert (ids == eb.EMB_ID_ABSENT).any()
        for mean in (False, True):
            pool = eb.EMB_POOL_MEAN if mean else eb.EMB_POOL_SUM
            out = torch.empty((w.B, w.T, w.D), dtype=torch.float32, device=DEV)
            eb.check(eb.emb_bag_forward(tabs.handle, _t(offsets), _t(ids), w.B, ids.size, pool,
                                        out), "forward")
            torch.cuda.synchronize()
            r, fl = o.forward(offsets, ids, w.B, mean)
            assert fl == 0
            S = (forward_S(offsets, ids, w.B, o.rows, lambda g: np.abs(o.read_rows(g)[0]), mean,
                           w.D) +
                 forward_S(offsets, ids, w.B, o.rows, bounds.weight_bound, mean, w.D) / REL)
            assert_within(out.cpu().numpy(), r, S, f"forward step {step}")
        grad = synth.gen_grad(w, step)
        ws, need = tabs.workspace(w.B, ids.size)
        eb.check(eb.emb_bag_backward_adagrad(tabs.handle, _t(offsets), _t(ids), w.B, ids.size,
                                             eb.EMB_POOL_SUM, _t(grad), w.lr, w.eps, ws, need),
                 "backward")
        rows_u, sums = abs_grad_sums(offsets, ids, w.B, o.rows, grad, False, w.D)
        assert bounds.step(o, rows_u, sums, w.lr, w.eps, lambda: o.backward_adagrad(
            offsets, ids, w.B, False, grad, w.lr, w.eps)) == 0
        assert status(tabs) == (eb.EMB_OK, 0)
    st, n_live = eb.emb_hash_n_live(tabs.handle, tabs.T)
    live = np.concatenate([np.arange(n) + int(np.sum(w.rows[:t])) for t, n in enumerate(n_live)])
    Wr, Gr = o.read_rows(live)
    bounds.check(tabs.weights[_t(live)].cpu().numpy(), tabs.accum[_t(live)].cpu().numpy(), Wr, Gr,
                 live, "admission, 3 steps")
