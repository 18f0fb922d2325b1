"""Property tests of the CPU oracle over random tiny CSR batches (hypothesis):
any number of tables, bag lengths 0..6 with empty bags, one-hot batches,
duplicate ids, sum and mean pooling.  Each property is checked against
something other than the oracle's own loops:

  * forward = A . W with the dense bag-by-row matrix A (numpy matmul in fp64);
  * sort/unique = numpy's stable argsort and np.unique (counts sum to nnz);
  * backward + Adagrad = A^T . grad followed by the textbook element-wise
    Adagrad step in fp64; rows outside the batch stay bit-identical.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import oracle as orc

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def batches(draw):
    T = draw(st.integers(1, 4))
    B = draw(st.integers(1, 6))
    D = draw(st.sampled_from([1, 2, 4, 5, 8]))
    rows = draw(st.lists(st.integers(1, 9), min_size=T, max_size=T))
    one_hot = draw(st.booleans())
    lens = [1] * (T * B) if one_hot else draw(
        st.lists(st.integers(0, 6), min_size=T * B, max_size=T * B))
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ids = np.empty(int(offsets[-1]), np.int64)
    for t in range(T):
        a, b = int(offsets[t * B]), int(offsets[(t + 1) * B])
        ids[a:b] = draw(st.lists(st.integers(0, rows[t] - 1), min_size=b - a, max_size=b - a))
    seed = draw(st.integers(0, 2**32))
    return T, B, D, np.array(rows, np.int64), offsets, ids, draw(st.booleans()), seed


def _dense_matrix(T, B, rows, offsets, ids, mean):
    """A[b, row] = c_b * (occurrences of row in bag b), b = t*B + s, global rows."""
    row_off = np.concatenate([[0], np.cumsum(rows)])
    A = np.zeros((T * B, int(row_off[-1])))
    for b in range(T * B):
        t = b // B
        L = offsets[b + 1] - offsets[b]
        for j in range(offsets[b], offsets[b + 1]):
            A[b, row_off[t] + ids[j]] += (1.0 / L) if mean else 1.0
    return A


def _tables(T, D, rows, seed):
    rng = np.random.default_rng(seed)
    n = int(rows.sum())
    W = rng.standard_normal((n, D)).astype(np.float32)
    G = (0.1 + rng.random((n, D))).astype(np.float32)
    o = orc.Oracle(rows, D)
    o.set_dense(W, G)
    return o, W, G


@SETTINGS
@given(batches())
def test_forward_is_dense_matrix_product(case):
    T, B, D, rows, offsets, ids, mean, seed = case
    o, W, _ = _tables(T, D, rows, seed)
    out, flags = o.forward(offsets, ids, B, mean)
    assert flags == 0
    A = _dense_matrix(T, B, rows, offsets, ids, mean)
    ref = (A @ W.astype(np.float64)).reshape(T, B, D).transpose(1, 0, 2)
    # one fp32 rounding of an fp64 sum
    np.testing.assert_allclose(out, ref, rtol=2 ** -23, atol=1e-30)


@SETTINGS
@given(batches())
def test_sort_unique_matches_numpy(case):
    T, B, D, rows, offsets, ids, mean, seed = case
    o = orc.Oracle(rows, D)
    r = o.sort_unique(offsets, ids, B)
    row_off = np.concatenate([[0], np.cumsum(rows)])
    t_of = np.repeat(np.arange(T * B), np.diff(offsets)) // B
    keys = row_off[t_of] + ids
    perm = np.argsort(keys, kind="stable")
    np.testing.assert_array_equal(r["perm"], perm)
    np.testing.assert_array_equal(r["sorted_rows"], keys[perm])
    u, inv, cnt = np.unique(keys, return_inverse=True, return_counts=True)
    np.testing.assert_array_equal(r["unique"], u)
    np.testing.assert_array_equal(r["counts"], cnt)
    np.testing.assert_array_equal(r["inverse"], inv)
    assert int(r["counts"].sum()) == ids.size
    np.testing.assert_array_equal(r["seg_off"], np.concatenate([[0], np.cumsum(cnt)]))


@SETTINGS
@given(batches(), st.sampled_from([0.01, 0.1]))
def test_backward_adagrad_is_dense_gradient_then_adagrad(case, lr):
    T, B, D, rows, offsets, ids, mean, seed = case
    o, W, G = _tables(T, D, rows, seed)
    grad = np.random.default_rng(seed + 1).standard_normal((B, T, D)).astype(np.float32)
    eps = 1e-6
    assert o.backward_adagrad(offsets, ids, B, mean, grad, lr, eps) == 0
    A = _dense_matrix(T, B, rows, offsets, ids, mean)
    g = A.T @ grad.transpose(1, 0, 2).reshape(T * B, D).astype(np.float64)
    touched = np.nonzero(A.sum(axis=0) > 0)[0]
    all_rows = np.arange(int(rows.sum()))
    W1, G1 = o.read_rows(all_rows)
    untouched = np.setdiff1d(all_rows, touched)
    assert np.array_equal(W1[untouched], W[untouched])
    assert np.array_equal(G1[untouched], G[untouched])
    gt = g[touched]
    G_ref = G[touched].astype(np.float64) + gt * gt
    # the accumulator is rounded to fp32 before the step uses it
    G_ref32 = G_ref.astype(np.float32)
    W_ref = W[touched].astype(np.float64) - lr * gt / (np.sqrt(G_ref32.astype(np.float64)) + eps)
    np.testing.assert_allclose(G1[touched], G_ref, rtol=3 * 2 ** -24, atol=1e-30)
    np.testing.assert_allclose(W1[touched], W_ref, rtol=3 * 2 ** -24, atol=2e-7 * lr)
    assert np.all(np.abs(W1[touched] - W[touched]) <= lr * (1 + 1e-6))
