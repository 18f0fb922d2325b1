"""Shared test helpers: error bounds for fp32 comparisons and GPU/oracle setup.

Tolerance rule for every fp32 output:  |gpu - oracle| <= 1e-5 * S + 1e-6, with
S the sum of absolute values of the terms that make the output (first-order
error propagation):
  pooled output       S = c_b * sum_j |W[row_j, d]|
  accumulator G'      S = |G| + (sum_k c_k |grad_k, d|)^2
  weight w'           S = |w| + lr * (sum_k c_k |grad_k, d|) / (sqrt(G') + eps)
  new hashed row      S = |w|
The oracle accumulates in fp64 and rounds once, so the bound is spent on the
GPU's fp32 summation order alone.
"""
import numpy as np

REL, ABS = 1e-5, 1e-6


def assert_within(gpu, ref, S, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    S = np.asarray(S, np.float64)
    err = np.abs(gpu - ref)
    bound = REL * S + ABS
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside 1e-5*S+1e-6; first {idx.tolist()}: "
            f"gpu {gpu[bad][:5]} ref {ref[bad][:5]} S {S[bad][:5]}")


def occurrence_rows(offsets, ids, B, rows):
    """Table, global row and grad-row index (s*T + t) of every occurrence."""
    rows = np.asarray(rows, np.int64)
    T = rows.size
    row_off = np.concatenate([[0], np.cumsum(rows)])
    lens = np.diff(offsets)
    bag = np.repeat(np.arange(T * B, dtype=np.int64), lens)
    t = bag // B
    s = bag % B
    valid = (ids >= 0) & (ids < rows[t])
    grow = np.where(valid, row_off[t] + ids, -1)
    scale = 1.0 / np.maximum(lens, 1)
    return t, grow, s * T + t, scale[bag], valid


def abs_grad_sums(offsets, ids, B, rows, grad, pool_mean, D):
    """For every touched global row: sum_k c_k |grad_k| (float64 [U, D]) and the rows."""
    _, grow, gr, sc, valid = occurrence_rows(offsets, ids, B, rows)
    r = grow[valid]
    order = np.argsort(r, kind="stable")
    r = r[order]
    g = np.abs(grad.reshape(-1, D)[gr[valid][order]])
    if pool_mean:
        g = g * sc[valid][order, None].astype(np.float32)
    uniq, start = np.unique(r, return_index=True)
    sums = np.add.reduceat(g.astype(np.float64), start, axis=0) if r.size else np.zeros((0, D))
    return uniq, sums


def forward_S(offsets, ids, B, rows, W_rows_of, pool_mean, D):
    """S for every pooled output: c_b * sum |W[row_j]| ([B, T, D]); W_rows_of(grows)->values.

    Occurrences are in CSR order, so each bag's terms are one contiguous run.
    """
    rows = np.asarray(rows, np.int64)
    T = rows.size
    t, grow, gr, sc, valid = occurrence_rows(offsets, ids, B, rows)
    vals = np.zeros((ids.size, D), np.float32)
    if valid.any():
        vals[valid] = np.abs(W_rows_of(grow[valid]))
    lens = np.diff(offsets)
    nonempty = lens > 0
    S_bag = np.zeros((T * B, D), np.float64)
    if ids.size:
        sums = np.add.reduceat(vals.astype(np.float64), offsets[:-1][nonempty], axis=0)
        S_bag[nonempty] = sums
    if pool_mean:
        S_bag[nonempty] /= lens[nonempty, None]
    # table-major bags -> [B, T, D]
    return S_bag.reshape(T, B, D).transpose(1, 0, 2)
