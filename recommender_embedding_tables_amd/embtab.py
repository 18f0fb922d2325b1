"""ctypes binding of libembtab.so, the gfx950 sparse embedding library.

Argument marshalling only: every function here has the name of a C entry point
of include/embtab.h and forwards device pointers (torch tensors) and sizes to
it.  All computation runs in the library's HIP kernels; importing this module
fails when the library has not been built.

Status codes are returned as ints (EMB_OK = 0); `check(status)` raises.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libembtab.so")

EMB_OK = 0
EMB_ERR_INVALID_ARG = 1
EMB_ERR_UNSUPPORTED = 2
EMB_ERR_WORKSPACE = 3
EMB_ERR_OUT_OF_RANGE = 4
EMB_ERR_BAD_OFFSETS = 5
EMB_ERR_RESERVED_KEY = 6
EMB_ERR_TABLE_FULL = 7
EMB_ERR_HIP = 8
EMB_ERR_CACHE_FULL = 9

EMB_FLAG_OUT_OF_RANGE = 1
EMB_FLAG_BAD_OFFSETS = 2
EMB_FLAG_RESERVED_KEY = 4
EMB_FLAG_TABLE_FULL = 8
EMB_FLAG_CACHE_FULL = 32

EMB_CACHE_WAYS = 16
EMB_NOALLOC_SCRATCH_BYTES = 64 << 20
EMB_PERIOD_FRESH = 0xFFFFFFFF
EMB_ID_ABSENT = -2

EMB_POOL_SUM = 0
EMB_POOL_MEAN = 1

EMB_EMPTY_KEY = 0xFFFFFFFFFFFFFFFF

EXPORTED = [
    "emb_state_bytes", "emb_hash_bytes", "emb_workspace_bytes", "emb_table_create",
    "emb_table_destroy", "emb_hash_find_or_insert", "emb_bag_forward",
    "emb_bag_backward_adagrad", "emb_bag_backward_adagrad_noalloc", "emb_status_sync",
    "emb_hash_n_live", "emb_hash_export",
    "emb_debug_sort_unique", "emb_status_string", "emb_set_phase_events", "emb_bag_prepare",
    "emb_bag_backward_adagrad_prepared", "emb_bag_forward_prepared", "emb_cache_state_bytes",
    "emb_table_create_tiered", "emb_cache_flush", "emb_cache_stats",
    "emb_bag_backward_adagrad_decay_prepared", "emb_hash_find_or_insert_admit",
    "emb_hash_evict_workspace_bytes", "emb_hash_evict", "emb_hash_free_rows",
    "emb_interact_out_dim", "emb_bag_forward_interact", "emb_interact_backward",
    "emb_bag_prepare_ids", "emb_cache_prepare", "emb_stream_copy", "emb_stream_fill",
    "emb_stream_read_sink_floats", "emb_stream_read", "emb_quantize_rows_int8",
    "emb_dequantize_rows_int8", "emb_bag_forward_prepared_int8",
    "emb_bag_backward_adagrad_prepared_int8",
]

EMB_PHASE_FORWARD, EMB_PHASE_KEYS, EMB_PHASE_SORT, EMB_PHASE_UNIQUE = 0, 1, 2, 3
EMB_PHASE_REDUCE, EMB_PHASE_FIXUP, EMB_PHASE_HASH, EMB_PHASE_CACHE = 4, 5, 6, 7
EMB_NUM_PHASES = 8
PHASE_NAMES = ["forward", "keys", "sort", "unique", "reduce_adagrad", "fixup", "hash",
               "cache_move"]


class emb_table_desc_t(C.Structure):
    _fields_ = [
        ("num_tables", C.c_int32),
        ("dim", C.c_int32),
        ("rows_per_table", C.c_void_p),
        ("weights", C.c_void_p),
        ("accum", C.c_void_p),
        ("state", C.c_void_p),
        ("hashed", C.c_int32),
        ("hash_capacity", C.c_int64),
        ("max_load", C.c_float),
        ("hash_slots", C.c_void_p),
        ("seed", C.c_uint64),
        ("init_lo", C.c_float),
        ("init_hi", C.c_float),
        ("init_std", C.c_float),
        ("accum_init", C.c_float),
        ("init_storage", C.c_int32),
        ("free_rows", C.c_void_p),
    ]


class emb_tier_desc_t(C.Structure):
    _fields_ = [
        ("host_weights", C.c_void_p),
        ("host_accum", C.c_void_p),
        ("cache_rows", C.c_int64),
        ("cache_state", C.c_void_p),
    ]


class EmbError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {emb_status_string(status)} (status {status})")


def _load():
    # torch first: its bundled HIP runtime then satisfies libembtab.so's
    # libamdhip64 dependency, so streams and events from torch and the
    # library's launches live in one runtime instance.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python recommender_embedding_tables_amd/build.py`")
    lib = C.CDLL(LIB_PATH)
    P, i32, i64, u32, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_float, C.c_size_t
    sig = {
        "emb_state_bytes": (sz, [i32]),
        "emb_hash_bytes": (sz, [i32, i64]),
        "emb_workspace_bytes": (sz, [P, i64, i64]),
        "emb_table_create": (i32, [C.POINTER(emb_table_desc_t), P, C.POINTER(P)]),
        "emb_table_destroy": (i32, [P]),
        "emb_hash_find_or_insert": (i32, [P, P, P, i64, i64, P, P, sz, P]),
        "emb_hash_find_or_insert_admit": (i32, [P, P, P, i64, i64, P, C.c_uint32, P, P, sz, P]),
        "emb_hash_evict_workspace_bytes": (sz, [P]),
        "emb_interact_out_dim": (i64, [P]),
        "emb_bag_forward_interact": (i32, [P, P, P, i64, i64, i32, P, P, P]),
        "emb_interact_backward": (i32, [P, P, P, i64, i64, i32, P, P, P, P, P]),
        "emb_hash_evict": (i32, [P, P, C.c_uint32, P, P, sz, P]),
        "emb_hash_free_rows": (i32, [P, P, C.POINTER(i64)]),
        "emb_bag_forward": (i32, [P, P, P, i64, i64, i32, P, P, sz, P]),
        "emb_bag_backward_adagrad": (i32, [P, P, P, i64, i64, i32, P, f32, f32, P, sz, P]),
        "emb_bag_backward_adagrad_noalloc": (i32, [P, P, P, i64, i64, i32, P, f32, f32, P]),
        "emb_status_sync": (i32, [P, P, C.POINTER(u32)]),
        "emb_hash_n_live": (i32, [P, P, P]),
        "emb_hash_export": (i32, [P, i32, P, P]),
        "emb_debug_sort_unique": (i32, [P, P, P, i64, i64, P, P, P, P, P, P, P, P, sz, P]),
        "emb_status_string": (C.c_char_p, [i32]),
        "emb_set_phase_events": (i32, [P, P]),
        "emb_bag_prepare": (i32, [P, P, P, i64, i64, i32, P, sz, P]),
        "emb_bag_forward_prepared": (i32, [P, P, P, i64, i64, i32, P, P, sz, P]),
        "emb_bag_backward_adagrad_prepared": (i32, [P, i64, i64, i32, P, f32, f32, P, sz, P]),
        "emb_bag_backward_adagrad_decay_prepared": (i32, [P, i64, i64, i32, P, f32, f32, f32,
                                                          C.c_uint32, P, P, sz, P]),
        "emb_cache_state_bytes": (sz, [i64]),
        "emb_table_create_tiered": (i32, [C.POINTER(emb_table_desc_t),
                                          C.POINTER(emb_tier_desc_t), P, C.POINTER(P)]),
        "emb_cache_flush": (i32, [P, P]),
        "emb_bag_prepare_ids": (i32, [P, P, P, i64, i64, i32, P, sz, P]),
        "emb_cache_prepare": (i32, [P, i64, i64, P, sz, P]),
        "emb_cache_stats": (i32, [P, P, C.POINTER(i64), C.POINTER(i64), C.POINTER(i64)]),
        "emb_stream_copy": (i32, [P, P, sz, P]),
        "emb_stream_fill": (i32, [P, f32, sz, P]),
        "emb_stream_read_sink_floats": (sz, [sz]),
        "emb_stream_read": (i32, [P, sz, P, sz, P]),
        "emb_quantize_rows_int8": (i32, [P, i64, i32, P, P, P]),
        "emb_bag_forward_prepared_int8": (i32, [P, P, P, i64, i64, i32, P, P, P, sz, P]),
        "emb_bag_backward_adagrad_prepared_int8": (i32, [P, i64, i64, i32, P, P, f32, f32, P, sz,
                                                         P]),
        "emb_dequantize_rows_int8": (i32, [P, P, i64, i32, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def _ptr(x):
    """Device (or host) address of a torch tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def check(status: int, what: str = "embtab") -> None:
    if status != EMB_OK:
        raise EmbError(status, what)


def emb_status_string(status: int) -> str:
    return _lib.emb_status_string(status).decode()


def emb_state_bytes(num_tables: int) -> int:
    return int(_lib.emb_state_bytes(num_tables))


def emb_hash_bytes(num_tables: int, capacity: int) -> int:
    return int(_lib.emb_hash_bytes(num_tables, capacity))


def emb_workspace_bytes(handle, batch: int, nnz: int) -> int:
    return int(_lib.emb_workspace_bytes(handle, batch, nnz))


def emb_table_create(desc: emb_table_desc_t, stream=None):
    """Returns (status, handle)."""
    h = C.c_void_p()
    st = _lib.emb_table_create(C.byref(desc), _stream(stream), C.byref(h))
    return st, h.value


def emb_cache_state_bytes(cache_rows: int) -> int:
    return int(_lib.emb_cache_state_bytes(cache_rows))


def emb_table_create_tiered(desc: emb_table_desc_t, tier: emb_tier_desc_t, stream=None):
    """Returns (status, handle)."""
    h = C.c_void_p()
    st = _lib.emb_table_create_tiered(C.byref(desc), C.byref(tier), _stream(stream), C.byref(h))
    return st, h.value


def emb_bag_prepare_ids(handle, offsets, ids, batch, nnz, pool, ws, ws_bytes,
                        stream=None) -> int:
    return _lib.emb_bag_prepare_ids(handle, _ptr(offsets), _ptr(ids), batch, nnz, pool, _ptr(ws),
                                    ws_bytes, _stream(stream))


def emb_cache_prepare(handle, batch, nnz, ws, ws_bytes, stream=None) -> int:
    return _lib.emb_cache_prepare(handle, batch, nnz, _ptr(ws), ws_bytes, _stream(stream))


def emb_cache_flush(handle, stream=None) -> int:
    return _lib.emb_cache_flush(handle, _stream(stream))


def emb_cache_stats(handle, stream=None):
    """Returns (status, lookups, misses, write-backs)."""
    a, b, c = C.c_int64(0), C.c_int64(0), C.c_int64(0)
    st = _lib.emb_cache_stats(handle, _stream(stream), C.byref(a), C.byref(b), C.byref(c))
    return st, int(a.value), int(b.value), int(c.value)


def emb_table_destroy(handle) -> int:
    return _lib.emb_table_destroy(handle)


def emb_hash_find_or_insert(handle, offsets, keys, batch, nnz, ids_out, ws, ws_bytes,
                            stream=None) -> int:
    return _lib.emb_hash_find_or_insert(handle, _ptr(offsets), _ptr(keys), batch, nnz,
                                        _ptr(ids_out), _ptr(ws), ws_bytes, _stream(stream))


def emb_hash_find_or_insert_admit(handle, offsets, keys, batch, nnz, ids_out, min_count,
                                  key_counts, ws, ws_bytes, stream=None) -> int:
    return _lib.emb_hash_find_or_insert_admit(handle, _ptr(offsets), _ptr(keys), batch, nnz,
                                              _ptr(ids_out), min_count, _ptr(key_counts),
                                              _ptr(ws), ws_bytes, _stream(stream))


def emb_interact_out_dim(handle) -> int:
    return int(_lib.emb_interact_out_dim(handle))


def emb_bag_forward_interact(handle, offsets, ids, batch, nnz, pool, dense, out,
                             stream=None) -> int:
    return _lib.emb_bag_forward_interact(handle, _ptr(offsets), _ptr(ids), batch, nnz, pool,
                                         _ptr(dense), _ptr(out), _stream(stream))


def emb_interact_backward(handle, offsets, ids, batch, nnz, pool, dense, grad_out, grad_dense,
                          grad_pooled, stream=None) -> int:
    return _lib.emb_interact_backward(handle, _ptr(offsets), _ptr(ids), batch, nnz, pool,
                                      _ptr(dense), _ptr(grad_out), _ptr(grad_dense),
                                      _ptr(grad_pooled), _stream(stream))


def emb_hash_evict_workspace_bytes(handle) -> int:
    return int(_lib.emb_hash_evict_workspace_bytes(handle))


def emb_hash_evict(handle, row_last_used, before, key_counts, ws, ws_bytes, stream=None) -> int:
    return _lib.emb_hash_evict(handle, _ptr(row_last_used), before, _ptr(key_counts), _ptr(ws),
                               ws_bytes, _stream(stream))


def emb_hash_free_rows(handle, num_tables, stream=None):
    """Returns (status, [rows queued per table])."""
    arr = (C.c_int64 * num_tables)()
    st = _lib.emb_hash_free_rows(handle, _stream(stream), arr)
    return st, list(arr)


def emb_bag_forward(handle, offsets, ids, batch, nnz, pool, out, ws=None, ws_bytes=0,
                    stream=None) -> int:
    return _lib.emb_bag_forward(handle, _ptr(offsets), _ptr(ids), batch, nnz, pool, _ptr(out),
                                _ptr(ws), ws_bytes, _stream(stream))


def emb_bag_backward_adagrad(handle, offsets, ids, batch, nnz, pool, grad_out, lr, eps, ws,
                             ws_bytes, stream=None) -> int:
    return _lib.emb_bag_backward_adagrad(handle, _ptr(offsets), _ptr(ids), batch, nnz, pool,
                                         _ptr(grad_out), lr, eps, _ptr(ws), ws_bytes,
                                         _stream(stream))


def emb_bag_backward_adagrad_noalloc(handle, offsets, ids, batch, nnz, pool, grad_out, lr, eps,
                                     stream=None) -> int:
    return _lib.emb_bag_backward_adagrad_noalloc(handle, _ptr(offsets), _ptr(ids), batch, nnz,
                                                 pool, _ptr(grad_out), lr, eps, _stream(stream))


def emb_bag_prepare(handle, offsets, ids, batch, nnz, pool, ws, ws_bytes, stream=None) -> int:
    return _lib.emb_bag_prepare(handle, _ptr(offsets), _ptr(ids), batch, nnz, pool, _ptr(ws),
                                ws_bytes, _stream(stream))


def emb_bag_forward_prepared(handle, offsets, ids, batch, nnz, pool, out, ws, ws_bytes,
                             stream=None) -> int:
    return _lib.emb_bag_forward_prepared(handle, _ptr(offsets), _ptr(ids), batch, nnz, pool,
                                         _ptr(out), _ptr(ws), ws_bytes, _stream(stream))


def emb_bag_backward_adagrad_prepared(handle, batch, nnz, pool, grad_out, lr, eps, ws, ws_bytes,
                                      stream=None) -> int:
    return _lib.emb_bag_backward_adagrad_prepared(handle, batch, nnz, pool, _ptr(grad_out), lr,
                                                  eps, _ptr(ws), ws_bytes, _stream(stream))


def emb_bag_backward_adagrad_decay_prepared(handle, batch, nnz, pool, grad_out, lr, eps, rho,
                                            period, row_periods, ws, ws_bytes,
                                            stream=None) -> int:
    return _lib.emb_bag_backward_adagrad_decay_prepared(
        handle, batch, nnz, pool, _ptr(grad_out), lr, eps, rho, period, _ptr(row_periods),
        _ptr(ws), ws_bytes, _stream(stream))


def emb_status_sync(handle, stream=None):
    """Returns (status, flag bits)."""
    f = C.c_uint32(0)
    st = _lib.emb_status_sync(handle, _stream(stream), C.byref(f))
    return st, int(f.value)


def emb_hash_n_live(handle, num_tables, stream=None):
    arr = (C.c_int64 * num_tables)()
    st = _lib.emb_hash_n_live(handle, _stream(stream), C.cast(arr, C.c_void_p))
    return st, [int(v) for v in arr]


def emb_hash_export(handle, table, key_of_row, stream=None) -> int:
    return _lib.emb_hash_export(handle, table, _ptr(key_of_row), _stream(stream))


def emb_set_phase_events(handle, events) -> int:
    """events: None, or 2 * EMB_NUM_PHASES raw hipEvent_t addresses (0 = skip)."""
    if events is None:
        return _lib.emb_set_phase_events(handle, None)
    arr = (C.c_void_p * (2 * EMB_NUM_PHASES))(*[e or None for e in events])
    return _lib.emb_set_phase_events(handle, C.cast(arr, C.c_void_p))


def emb_debug_sort_unique(handle, offsets, ids, batch, nnz, sorted_rows, perm, unique, counts,
                          seg_off, inverse, num_unique, ws, ws_bytes, stream=None) -> int:
    return _lib.emb_debug_sort_unique(handle, _ptr(offsets), _ptr(ids), batch, nnz,
                                      _ptr(sorted_rows), _ptr(perm), _ptr(unique), _ptr(counts),
                                      _ptr(seg_off), _ptr(inverse), _ptr(num_unique), _ptr(ws),
                                      ws_bytes, _stream(stream))


class EmbTables:
    """Owns the device storage of one table set (weights, accumulators, state,
    hash slots) as torch tensors and the library handle over it.

    Storage allocation is torch's; every computation is a library call.
    """

    def __init__(self, rows_per_table, dim, *, hashed=False, hash_capacity=0, max_load=0.625,
                 seed=0, init_lo=-0.05, init_hi=0.05, init_std=0.01, accum_init=0.1,
                 device="cuda", stream=None, storage=None, cache_rows=0,
                 host_storage=None):
        import torch
        self.rows = [int(r) for r in rows_per_table]
        self.T = len(self.rows)
        self.D = int(dim)
        self.total_rows = sum(self.rows)
        self.hashed = bool(hashed)
        self.hash_capacity = int(hash_capacity)
        dev = torch.device(device)
        self.tiered = cache_rows > 0
        if self.tiered:
            if host_storage is not None:  # attach: the host rows of an earlier (flushed) handle
                self.host_weights, self.host_accum = host_storage
            else:
                # the table in pinned host memory; weights / accum below are the HBM cache
                self.host_weights = torch.empty((self.total_rows, self.D), dtype=torch.float32,
                                                pin_memory=True)
                self.host_accum = torch.empty_like(self.host_weights, pin_memory=True)
            self.cache_state = torch.empty(max(emb_cache_state_bytes(cache_rows), 256),
                                           dtype=torch.uint8, device=dev)
        if storage is None:
            nrows = cache_rows if self.tiered else self.total_rows
            self.weights = torch.empty((nrows, self.D), dtype=torch.float32, device=dev)
            self.accum = torch.empty_like(self.weights)
            self.state = torch.zeros(emb_state_bytes(self.T), dtype=torch.uint8, device=dev)
            hb = emb_hash_bytes(self.T, self.hash_capacity) if hashed else 0
            self.slots = torch.empty(max(hb, 16), dtype=torch.uint8, device=dev) if hashed else None
            # free-row queue of emb_hash_evict: 4 bytes per row
            self.free_rows = (torch.empty(self.total_rows, dtype=torch.int32, device=dev)
                              if hashed else None)
            init = 1
        else:
            self.weights, self.accum, self.state, self.slots = storage[:4]
            self.free_rows = storage[4] if len(storage) > 4 else None
            init = 0
        self._rows_c = (C.c_int64 * self.T)(*self.rows)
        d = emb_table_desc_t()
        d.num_tables = self.T
        d.dim = self.D
        d.rows_per_table = C.cast(self._rows_c, C.c_void_p)
        d.weights = self.weights.data_ptr()
        d.accum = self.accum.data_ptr()
        d.state = self.state.data_ptr()
        d.hashed = 1 if hashed else 0
        d.hash_capacity = self.hash_capacity
        d.max_load = max_load
        d.hash_slots = self.slots.data_ptr() if hashed else None
        d.free_rows = self.free_rows.data_ptr() if self.free_rows is not None else None
        d.seed = seed
        d.init_lo = init_lo
        d.init_hi = init_hi
        d.init_std = init_std
        d.accum_init = accum_init
        d.init_storage = init
        if self.tiered:
            tier = emb_tier_desc_t()
            tier.host_weights = self.host_weights.data_ptr()
            tier.host_accum = self.host_accum.data_ptr()
            tier.cache_rows = int(cache_rows)
            tier.cache_state = self.cache_state.data_ptr()
            st, self.handle = emb_table_create_tiered(d, tier, stream)
            check(st, "emb_table_create_tiered")
        else:
            st, self.handle = emb_table_create(d, stream)
            check(st, "emb_table_create")
        self._ws = None

    def close(self):
        if getattr(self, "handle", None):
            emb_table_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, batch, nnz):
        """A torch uint8 workspace large enough for (batch, nnz), reused when possible."""
        import torch
        need = emb_workspace_bytes(self.handle, batch, nnz)
        if need == 0:
            raise EmbError(EMB_ERR_INVALID_ARG, "emb_workspace_bytes")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need + 256, dtype=torch.uint8, device=self.weights.device)
        return self._ws, need


def emb_stream_copy(dst, src, nbytes, stream=None) -> int:
    return _lib.emb_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream))


def emb_stream_fill(dst, value, nbytes, stream=None) -> int:
    return _lib.emb_stream_fill(_ptr(dst), value, nbytes, _stream(stream))


def emb_stream_read_sink_floats(nbytes) -> int:
    return int(_lib.emb_stream_read_sink_floats(nbytes))


def emb_stream_read(src, nbytes, sink, sink_floats, stream=None) -> int:
    return _lib.emb_stream_read(_ptr(src), nbytes, _ptr(sink), sink_floats, _stream(stream))


def emb_quantize_rows_int8(x, rows, dim, codes, scales, stream=None) -> int:
    return _lib.emb_quantize_rows_int8(_ptr(x), rows, dim, _ptr(codes), _ptr(scales),
                                       _stream(stream))


def emb_bag_forward_prepared_int8(handle, offsets, ids, batch, nnz, pool, codes, scales, ws,
                                  ws_bytes, stream=None) -> int:
    return _lib.emb_bag_forward_prepared_int8(handle, _ptr(offsets), _ptr(ids), batch, nnz,
                                              pool, _ptr(codes), _ptr(scales), _ptr(ws),
                                              ws_bytes, _stream(stream))


def emb_bag_backward_adagrad_prepared_int8(handle, batch, nnz, pool, grad_codes, grad_scales, lr,
                                           eps, ws, ws_bytes, stream=None) -> int:
    return _lib.emb_bag_backward_adagrad_prepared_int8(handle, batch, nnz, pool,
                                                       _ptr(grad_codes), _ptr(grad_scales), lr,
                                                       eps, _ptr(ws), ws_bytes, _stream(stream))


def emb_dequantize_rows_int8(codes, scales, rows, dim, y, stream=None) -> int:
    return _lib.emb_dequantize_rows_int8(_ptr(codes), _ptr(scales), rows, dim, _ptr(y),
                                         _stream(stream))
