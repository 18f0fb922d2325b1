"""ctypes wrapper of the CPU oracle (oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It marshals numpy
arrays into the plain C calls of liboracle.so and holds no arithmetic of its
own.  Error bits returned by the calls: 1 id out of range, 2 bad offsets,
4 reserved key, 8 table full.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

ERR_OUT_OF_RANGE = 1
ERR_BAD_OFFSETS = 2
ERR_RESERVED_KEY = 4
ERR_TABLE_FULL = 8

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b  # noqa: F401  (package-relative when imported as oracle.oracle)
        _b.build()
    lib = C.CDLL(LIB_PATH)
    P = C.c_void_p
    i64, i32, u64, f32 = C.c_int64, C.c_int32, C.c_uint64, C.c_float
    sig = {
        "orc_splitmix64": (u64, [u64]),
        "orc_draw_bits": (u64, [u64, i64, u64, u64]),
        "orc_init_uniform": (f32, [u64, i64, i64, i64, f32, f32]),
        "orc_init_normal": (f32, [u64, i64, u64, i64, f32]),
        "orc_create": (P, [i64, i64, P, i32, u64, f32, f32, f32, f32]),
        "orc_destroy": (None, [P]),
        "orc_set_slot_limit": (i32, [P, i64]),
        "orc_set_dense": (i32, [P, P, P]),
        "orc_forward": (i32, [P, P, P, i64, i64, i32, P]),
        "orc_sort_unique": (i32, [P, P, P, i64, i64, P, P, P, P, P, P, P]),
        "orc_backward_adagrad": (i32, [P, P, P, i64, i64, i32, P, f32, f32]),
        "orc_backward_adagrad_decay": (i32, [P, P, P, i64, i64, i32, P, f32, f32, f32,
                                             C.c_uint32]),
        "orc_read_rows": (i32, [P, P, i64, P, P]),
        "orc_interact_forward": (i32, [P, P, P, i64, i64, i32, P, P]),
        "orc_interact_backward": (i32, [P, P, P, i64, i64, i32, P, P, P, P]),
        "orc_read_periods": (i32, [P, P, i64, P]),
        "orc_touched_count": (i64, [P]),
        "orc_touched_rows": (i64, [P, P]),
        "orc_hash_find_or_insert": (i32, [P, P, P, i64, i64, P]),
        "orc_hash_find_or_insert_admit": (i32, [P, P, P, i64, i64, P, C.c_uint32]),
        "orc_admission_count": (u64, [P, i64, u64]),
        "orc_n_live": (i64, [P, i64]),
        "orc_hash_evict": (i64, [P, P, C.c_uint32]),
        "orc_free_rows": (i64, [P, i64]),
        "orc_hash_export": (i64, [P, i64, P, P, i64]),
        "orc_quantize_rows_int8": (i32, [P, i64, i64, P, P]),
        "orc_dequantize_rows_int8": (i32, [P, P, i64, i64, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


def _arr(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def splitmix64(x):
    return int(_load().orc_splitmix64(C.c_uint64(x)))


def draw_bits(seed, t, r, i):
    return int(_load().orc_draw_bits(seed, t, r, i))


def quantize_rows_int8(x):
    """x: [rows, D] fp32 -> (codes int8 [rows, D], scales fp32 [rows])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, D = x.shape
    codes = np.empty((rows, D), np.int8)
    scales = np.empty(rows, np.float32)
    assert _load().orc_quantize_rows_int8(_p(x), rows, D, _p(codes), _p(scales)) == 0
    return codes, scales


def dequantize_rows_int8(codes, scales):
    """codes int8 [rows, D], scales fp32 [rows] -> fp32 [rows, D]."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    rows, D = codes.shape
    y = np.empty((rows, D), np.float32)
    assert _load().orc_dequantize_rows_int8(_p(codes), _p(scales), rows, D, _p(y)) == 0
    return y


def init_uniform(seed, t, row, d, lo, hi):
    return float(np.float32(_load().orc_init_uniform(seed, t, row, d, lo, hi)))


def init_normal(seed, t, key, d, std):
    return float(np.float32(_load().orc_init_normal(seed, t, key, d, std)))


class Oracle:
    """Sequential model of a set of T tables of dim D (dense or hashed)."""

    def __init__(self, rows_per_table, dim, hashed=False, seed=0, init_lo=-0.05,
                 init_hi=0.05, init_std=0.01, accum_init=0.1, slot_limit=None):
        lib = _load()
        self.rows = _arr(rows_per_table, np.int64)
        self.T = int(self.rows.size)
        self.D = int(dim)
        self.row_off = np.concatenate([[0], np.cumsum(self.rows)]).astype(np.int64)
        self.hashed = bool(hashed)
        self._h = lib.orc_create(self.T, self.D, _p(self.rows), int(hashed), C.c_uint64(seed),
                                 init_lo, init_hi, init_std, accum_init)
        if not self._h:
            raise ValueError("oracle: bad table description")
        if slot_limit is not None and lib.orc_set_slot_limit(self._h, int(slot_limit)) != 0:
            raise ValueError("oracle: bad slot limit")

    def close(self):
        if self._h:
            _load().orc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_dense(self, W, G):
        W = _arr(W, np.float32)
        G = _arr(G, np.float32)
        n = int(self.row_off[-1]) * self.D
        assert W.size == n and G.size == n
        _load().orc_set_dense(self._h, _p(W), _p(G))

    def forward(self, offsets, ids, batch, pool_mean):
        offsets = _arr(offsets, np.int64)
        ids = _arr(ids, np.int64)
        out = np.zeros((batch, self.T, self.D), np.float32)
        flags = _load().orc_forward(self._h, _p(offsets), _p(ids), batch, ids.size,
                                    int(bool(pool_mean)), _p(out))
        return out, int(flags)

    def sort_unique(self, offsets, ids, batch):
        offsets = _arr(offsets, np.int64)
        ids = _arr(ids, np.int64)
        n = ids.size
        sorted_rows = np.zeros(n, np.uint32)
        perm = np.zeros(n, np.uint32)
        unique = np.zeros(n, np.uint32)
        counts = np.zeros(n, np.uint32)
        seg_off = np.zeros(n + 1, np.uint32)
        inverse = np.zeros(n, np.uint32)
        nu = np.zeros(1, np.int64)
        flags = _load().orc_sort_unique(self._h, _p(offsets), _p(ids), batch, n, _p(sorted_rows),
                                        _p(perm), _p(unique), _p(counts), _p(seg_off),
                                        _p(inverse), _p(nu))
        U = int(nu[0])
        return dict(sorted_rows=sorted_rows, perm=perm, unique=unique[:U], counts=counts[:U],
                    seg_off=seg_off[:U + 1], inverse=inverse, num_unique=U, flags=int(flags))

    def backward_adagrad(self, offsets, ids, batch, pool_mean, grad_out, lr, eps):
        offsets = _arr(offsets, np.int64)
        ids = _arr(ids, np.int64)
        grad_out = _arr(grad_out, np.float32)
        assert grad_out.size == batch * self.T * self.D
        return int(_load().orc_backward_adagrad(self._h, _p(offsets), _p(ids), batch, ids.size,
                                                int(bool(pool_mean)), _p(grad_out), lr, eps))

    def backward_adagrad_decay(self, offsets, ids, batch, pool_mean, grad_out, lr, eps, rho,
                               period):
        """Adagrad Decay: accumulators discounted by rho per period (lazily, at a
        row's next update), then the Adagrad step; the row's period becomes `period`."""
        offsets = _arr(offsets, np.int64)
        ids = _arr(ids, np.int64)
        grad_out = _arr(grad_out, np.float32)
        assert grad_out.size == batch * self.T * self.D
        return int(_load().orc_backward_adagrad_decay(
            self._h, _p(offsets), _p(ids), batch, ids.size, int(bool(pool_mean)), _p(grad_out),
            lr, eps, rho, int(period)))

    def read_periods(self, grows):
        grows = _arr(grows, np.int64)
        out = np.zeros(grows.size, np.uint32)
        if _load().orc_read_periods(self._h, _p(grows), grows.size, _p(out)) != 0:
            raise IndexError("oracle: row out of range")
        return out

    def interact_forward(self, offsets, ids, batch, pool_mean, dense):
        """DLRM dot interaction over [dense, pooled embeddings]: [B, D + (T+1)T/2]."""
        offsets, ids = _arr(offsets, np.int64), _arr(ids, np.int64)
        dense = _arr(dense, np.float32)
        P = (self.T + 1) * self.T // 2
        out = np.zeros((batch, self.D + P), np.float32)
        rc = _load().orc_interact_forward(self._h, _p(offsets), _p(ids), batch, ids.size,
                                          int(bool(pool_mean)), _p(dense), _p(out))
        return out, int(rc)

    def interact_backward(self, offsets, ids, batch, pool_mean, dense, grad_out):
        """Gradients of interact_forward: (grad_dense [B, D], grad_pooled [B, T, D])."""
        offsets, ids = _arr(offsets, np.int64), _arr(ids, np.int64)
        dense, grad_out = _arr(dense, np.float32), _arr(grad_out, np.float32)
        gd = np.zeros((batch, self.D), np.float32)
        gp = np.zeros((batch, self.T, self.D), np.float32)
        rc = _load().orc_interact_backward(self._h, _p(offsets), _p(ids), batch, ids.size,
                                           int(bool(pool_mean)), _p(dense), _p(grad_out),
                                           _p(gd), _p(gp))
        return gd, gp, int(rc)

    def read_rows(self, grows):
        grows = _arr(grows, np.int64)
        W = np.zeros((grows.size, self.D), np.float32)
        G = np.zeros((grows.size, self.D), np.float32)
        rc = _load().orc_read_rows(self._h, _p(grows), grows.size, _p(W), _p(G))
        if rc != 0:
            raise IndexError("oracle: row out of range")
        return W, G

    def touched_rows(self):
        n = int(_load().orc_touched_count(self._h))
        out = np.zeros(n, np.int64)
        _load().orc_touched_rows(self._h, _p(out))
        return out

    def find_or_insert(self, offsets, keys, batch):
        offsets = _arr(offsets, np.int64)
        keys = _arr(keys, np.uint64)
        ids = np.zeros(keys.size, np.int64)
        flags = _load().orc_hash_find_or_insert(self._h, _p(offsets), _p(keys), batch, keys.size,
                                                _p(ids))
        return ids, int(flags)

    def find_or_insert_admit(self, offsets, keys, batch, min_count):
        """Find-or-insert where a key gets a row once its occurrences (over
        calls) reach min_count; until then its ids are -2 (absent)."""
        offsets = _arr(offsets, np.int64)
        keys = _arr(keys, np.uint64)
        ids = np.zeros(keys.size, np.int64)
        flags = _load().orc_hash_find_or_insert_admit(self._h, _p(offsets), _p(keys), batch,
                                                      keys.size, _p(ids), int(min_count))
        return ids, int(flags)

    def evict(self, last_used, before):
        """Keys whose row (global index into last_used) was last used before
        `before` leave the map; their rows are handed out again later."""
        last_used = _arr(last_used, np.uint32)
        assert last_used.size == int(self.row_off[-1])
        return int(_load().orc_hash_evict(self._h, _p(last_used), int(before)))

    def free_rows(self, t):
        return int(_load().orc_free_rows(self._h, t))

    def admission_count(self, t, key):
        return int(_load().orc_admission_count(self._h, t, int(key)))

    def n_live(self, t):
        return int(_load().orc_n_live(self._h, t))

    def export(self, t):
        n = int(_load().orc_hash_export(self._h, t, None, None, 0))
        keys = np.zeros(n, np.uint64)
        rows = np.zeros(n, np.int64)
        _load().orc_hash_export(self._h, t, _p(keys), _p(rows), n)
        return keys, rows
