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


class StepBounds:
    """The per-step rule carried over several Adagrad steps (first-order error
    propagation), per element of every row:

      before the first step   e_W = e_G = 0 (the initial tables are bit-exact);
                              a hashed row given a key: e_W = REL*|w0| + ABS, e_G = 0
      step i on a row         a = sum_k c_k |grad_k| of the row in this step
        e_G <- e_G + REL*(|G_before| + a^2) + ABS
        e_W <- e_W + REL*(|w_before| + lr*a/(sqrt(G_after)+eps)) + ABS
                   + lr*a/(2*G_after^1.5) * e_G          (the step's sensitivity to G)
      rows a step does not touch keep their bounds.

    An input error passes into the next step with factor 1 (w' = w - ..., G' =
    G*df + g^2 with df <= 1), so the bounds add up along the oracle's own
    trajectory, read before and after each oracle step.  Only rows that carry
    a bound are stored (sorted global rows and their [n, D] bounds)."""

    def __init__(self, total_rows, D):
        self.D = int(D)
        self.rows = np.zeros(0, np.int64)
        self._eW = np.zeros((0, self.D))
        self._eG = np.zeros((0, self.D))

    def _positions(self, rows):
        """Positions of `rows` in the store, adding the missing ones (bound 0)."""
        rows = np.asarray(rows, np.int64)
        new = np.setdiff1d(rows, self.rows)
        if new.size:
            allr = np.concatenate([self.rows, new])
            order = np.argsort(allr, kind="stable")
            self.rows = allr[order]
            z = np.zeros((new.size, self.D))
            self._eW = np.concatenate([self._eW, z])[order]
            self._eG = np.concatenate([self._eG, z])[order]
        return np.searchsorted(self.rows, rows)

    def bounds_of(self, rows):
        """(e_W, e_G) of `rows` ([n, D] each); 0 for rows that carry none."""
        rows = np.asarray(rows, np.int64)
        eW = np.zeros((rows.size, self.D))
        eG = np.zeros((rows.size, self.D))
        if self.rows.size and rows.size:
            pos = np.minimum(np.searchsorted(self.rows, rows), self.rows.size - 1)
            hit = self.rows[pos] == rows
            eW[hit] = self._eW[pos[hit]]
            eG[hit] = self._eG[pos[hit]]
        return eW, eG

    def weight_bound(self, rows):
        return self.bounds_of(rows)[0]

    def assigned(self, o, rows):
        """Rows that just got a key: fresh initial values (within the rule)."""
        rows = np.asarray(rows, np.int64)
        if rows.size:
            W, _ = o.read_rows(rows)
            pos = self._positions(rows)
            self._eW[pos] = REL * np.abs(W.astype(np.float64)) + ABS
            self._eG[pos] = 0.0

    def step(self, o, rows_u, sums, lr, eps, oracle_step):
        """Runs oracle_step() (the oracle's update of rows_u) and carries the bounds."""
        rows_u = np.asarray(rows_u, np.int64)
        W0, G0 = o.read_rows(rows_u) if rows_u.size else (None, None)
        rc = oracle_step()
        if rows_u.size:
            W1, G1 = o.read_rows(rows_u)
            a = np.asarray(sums, np.float64)
            G1 = G1.astype(np.float64)
            pos = self._positions(rows_u)
            eG = self._eG[pos] + REL * (np.abs(G0.astype(np.float64)) + a * a) + ABS
            eW = (self._eW[pos] + ABS +
                  REL * (np.abs(W0.astype(np.float64)) + lr * a / (np.sqrt(G1) + eps)) +
                  lr * a / (2.0 * G1 ** 1.5) * eG)
            self._eG[pos] = eG
            self._eW[pos] = eW
        return rc

    def check(self, W_gpu, G_gpu, W_ref, G_ref, rows, what):
        eW, eG = self.bounds_of(rows)
        for name, g, r, e in (("weights", W_gpu, W_ref, eW), ("accumulators", G_gpu, G_ref, eG)):
            err = np.abs(np.asarray(g, np.float64) - np.asarray(r, np.float64))
            bad = err > e
            if bad.any():
                idx = np.argwhere(bad)[:5]
                raise AssertionError(
                    f"{what} {name}: {int(bad.sum())} of {bad.size} outside the carried bound; "
                    f"first {idx.tolist()}: err {err[bad][:5]} bound {e[bad][:5]}")


def key_rows(o):
    """{global row: key} of every live key of a hashed oracle."""
    m = {}
    for t in range(o.T):
        k, r = o.export(t)
        base = int(o.row_off[t])
        m.update({base + int(rr): int(kk) for kk, rr in zip(k, r)})
    return m


def rows_given_keys(before, after):
    """Global rows whose key in `after` is new (inserted, or reused after eviction)."""
    return np.array(sorted(r for r, k in after.items() if before.get(r) != k), np.int64)


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


# ------------------------------------------------------------ guard bands
GUARD_BYTES = 4096  # a multiple of 256: the guarded region keeps its alignment
CANARY = 0xA5


class Guarded:
    """A device buffer of `nbytes` (viewed as `shape` of `dtype`) with GUARD_BYTES
    canary bytes before and after it; check() asserts that no call wrote there."""

    def __init__(self, shape, dtype, device, nbytes=None):
        import torch
        if nbytes is None:
            nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = int(nbytes)
        self.buf = torch.full((2 * GUARD_BYTES + self.nbytes,), CANARY, dtype=torch.uint8,
                              device=device)
        inner = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes]
        self.t = inner.view(dtype).view(shape) if shape is not None else inner

    def check(self, what):
        head = self.buf[:GUARD_BYTES]
        tail = self.buf[GUARD_BYTES + self.nbytes:]
        ok = bool((head == CANARY).all()) and bool((tail == CANARY).all())
        assert ok, f"{what}: a call wrote outside its buffer (guard band changed)"
