"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any launch."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "embtab.h")

eb = pytest.importorskip("recommender_embedding_tables_amd.embtab",
                         reason="libembtab.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(emb_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    lib = C.CDLL(eb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(eb.EXPORTED) == names


def test_size_queries():
    assert eb.emb_state_bytes(0) == 0
    assert eb.emb_state_bytes(1) >= 256 + 8 * 4
    assert eb.emb_state_bytes(26) % 256 == 0
    assert eb.emb_hash_bytes(4, 1 << 25) == 4 * (1 << 25) * 16
    assert eb.emb_hash_bytes(4, 1000) == 0  # not a power of two
    assert eb.emb_hash_bytes(0, 1024) == 0
    assert eb.emb_workspace_bytes(None, 10, 10) == 0


def _desc(**kw):
    rows = kw.pop("rows", [100, 200])
    arr = (C.c_int64 * len(rows))(*rows)
    d = eb.emb_table_desc_t()
    d.num_tables = len(rows)
    d.dim = kw.pop("dim", 16)
    d.rows_per_table = C.cast(arr, C.c_void_p)
    # fake, aligned device addresses: with init_storage = 0 nothing is touched
    d.weights = kw.pop("weights", 0x10000000)
    d.accum = kw.pop("accum", 0x20000000)
    d.state = kw.pop("state", 0x30000000)
    d.hashed = kw.pop("hashed", 0)
    d.hash_capacity = kw.pop("hash_capacity", 0)
    d.max_load = kw.pop("max_load", 0.625)
    d.hash_slots = kw.pop("hash_slots", None)
    d.init_storage = 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d, arr


@pytest.mark.parametrize("kw,code", [
    (dict(dim=3), eb.EMB_ERR_INVALID_ARG),
    (dict(dim=0), eb.EMB_ERR_INVALID_ARG),
    (dict(dim=2048), eb.EMB_ERR_INVALID_ARG),
    (dict(rows=[0]), eb.EMB_ERR_INVALID_ARG),
    (dict(weights=None), eb.EMB_ERR_INVALID_ARG),
    (dict(weights=0x10000004), eb.EMB_ERR_INVALID_ARG),  # misaligned
    (dict(state=0x30000010), eb.EMB_ERR_INVALID_ARG),    # state needs 256-byte alignment
    (dict(rows=[2**31, 2**31]), eb.EMB_ERR_UNSUPPORTED),  # rows are 32-bit inside
    (dict(hashed=1, hash_capacity=1000, hash_slots=0x40000000), eb.EMB_ERR_INVALID_ARG),
    (dict(hashed=1, hash_capacity=1024, hash_slots=None), eb.EMB_ERR_INVALID_ARG),
    (dict(hashed=1, rows=[700], hash_capacity=1024, hash_slots=0x40000000),
     eb.EMB_ERR_INVALID_ARG),  # 700 rows > 0.625 * 1024
])
def test_create_rejects(kw, code):
    d, _keep = _desc(**kw)
    st, h = eb.emb_table_create(d, 0)
    assert st == code and h is None


def test_host_checks_on_attached_handle():
    d, _keep = _desc(rows=[1000, 24], dim=64)
    st, h = eb.emb_table_create(d, 0)
    assert st == eb.EMB_OK and h
    try:
        ws = eb.emb_workspace_bytes(h, 4096, 10000)
        assert ws > 0 and ws % 256 == 0
        assert eb.emb_workspace_bytes(h, 4096, 20000) > ws
        assert eb.emb_workspace_bytes(h, -1, 10) == 0
        fake = 0x50000000
        # workspace too small / missing / misaligned
        assert eb.emb_bag_backward_adagrad(h, fake, fake, 4096, 10000, 0, fake, 0.01, 1e-8,
                                           fake, ws - 1, 0) == eb.EMB_ERR_WORKSPACE
        assert eb.emb_bag_backward_adagrad(h, fake, fake, 4096, 10000, 0, fake, 0.01, 1e-8,
                                           None, ws, 0) == eb.EMB_ERR_WORKSPACE
        assert eb.emb_bag_backward_adagrad(h, fake, fake, 4096, 10000, 0, fake, 0.01, 1e-8,
                                           fake + 16, ws, 0) == eb.EMB_ERR_WORKSPACE
        # bad pool, null pointers, bad lr / eps
        assert eb.emb_bag_forward(h, fake, fake, 4096, 10000, 7, fake, stream=0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_forward(h, fake, fake, 4096, 10000, 0, None, stream=0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_forward(h, None, fake, 4096, 10000, 0, fake, stream=0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_forward(h, fake, None, 4096, 10000, 0, fake, stream=0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_forward(h, fake, fake, -1, 10000, 0, fake, stream=0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_forward(h, fake, fake, 4096, 10000, 0, fake + 4, stream=0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_backward_adagrad(h, fake, fake, 4096, 10000, 0, fake, float("nan"),
                                           1e-8, fake, ws, 0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_backward_adagrad(h, fake, fake, 4096, 10000, 0, fake, 0.01, -1.0,
                                           fake, ws, 0) == eb.EMB_ERR_INVALID_ARG
        # the split backward checks the same things
        assert eb.emb_bag_prepare(h, fake, fake, 4096, 10000, 0, fake, ws - 1,
                                  0) == eb.EMB_ERR_WORKSPACE
        assert eb.emb_bag_prepare(h, None, fake, 4096, 10000, 0, fake, ws,
                                  0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_prepare(h, fake, fake, 4096, 10000, 3, fake, ws,
                                  0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_backward_adagrad_prepared(h, 4096, 10000, 0, fake, 0.01, 1e-8, fake,
                                                    ws - 1, 0) == eb.EMB_ERR_WORKSPACE
        assert eb.emb_bag_backward_adagrad_prepared(h, 4096, 10000, 0, None, 0.01, 1e-8, fake,
                                                    ws, 0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_backward_adagrad_prepared(h, 4096, 10000, 0, fake, 0.01, float("inf"),
                                                    fake, ws, 0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_forward_prepared(h, fake, fake, 4096, 10000, 0, fake, fake, ws - 1,
                                           0) == eb.EMB_ERR_WORKSPACE
        assert eb.emb_bag_forward_prepared(h, fake, fake, 4096, 10000, 0, None, fake, ws,
                                           0) == eb.EMB_ERR_INVALID_ARG
        # the backward on the library's own buffer: a batch over the buffer, sizes
        # beyond the 32-bit indices and bad arguments fail before any launch
        lim = eb.EMB_NOALLOC_SCRATCH_BYTES
        assert eb.emb_workspace_bytes(h, 4096, 4_000_000) > lim
        assert eb.emb_bag_backward_adagrad_noalloc(None, fake, fake, 4096, 10000, 0, fake, 0.01,
                                                   1e-8, 0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_backward_adagrad_noalloc(h, fake, fake, 4096, 4_000_000, 0, fake, 0.01,
                                                   1e-8, 0) == eb.EMB_ERR_WORKSPACE
        assert eb.emb_bag_backward_adagrad_noalloc(h, fake, fake, 4096, 2**33, 0, fake, 0.01,
                                                   1e-8, 0) == eb.EMB_ERR_UNSUPPORTED
        assert eb.emb_bag_backward_adagrad_noalloc(h, fake, fake, 4096, 10000, 0, fake,
                                                   float("nan"), 1e-8,
                                                   0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_backward_adagrad_noalloc(h, fake, fake, 4096, 10000, 5, fake, 0.01,
                                                   1e-8, 0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_bag_backward_adagrad_noalloc(h, None, fake, 4096, 10000, 0, fake, 0.01,
                                                   1e-8, 0) == eb.EMB_ERR_INVALID_ARG
        # hash calls on a dense handle
        assert eb.emb_hash_find_or_insert(h, fake, fake, 4096, 10000, fake, fake, ws,
                                          0) == eb.EMB_ERR_UNSUPPORTED
        assert eb.emb_hash_export(h, 0, fake, 0) == eb.EMB_ERR_UNSUPPORTED
        assert eb.emb_hash_export(h, 5, fake, 0) == eb.EMB_ERR_INVALID_ARG
        # sizes beyond the 32-bit internal indices
        assert eb.emb_bag_forward(h, fake, fake, 4096, 2**33, 0, fake, stream=0) == eb.EMB_ERR_UNSUPPORTED
        # an empty batch is a no-op
        assert eb.emb_bag_forward(h, fake, fake, 0, 0, 0, fake, stream=0) == eb.EMB_OK
    finally:
        eb.emb_table_destroy(h)


def test_status_strings():
    assert eb.emb_status_string(eb.EMB_ERR_TABLE_FULL) == "table full"
    assert eb.emb_status_string(eb.EMB_OK) == "ok"
    assert eb.emb_status_string(99) == "unknown status"


def test_cache_state_bytes():
    W = eb.EMB_CACHE_WAYS
    for bad in (0, -W, W - 1, W + 1, 3 * W, 48 * W):
        assert eb.emb_cache_state_bytes(bad) == 0, bad
    small, big = eb.emb_cache_state_bytes(W), eb.emb_cache_state_bytes(1024 * W)
    assert small > 0 and big > small and big % 256 == 0
    # per slot at least the row it holds and the step it was last used at
    assert big >= 1024 * W * 8


def _tier(**kw):
    t = eb.emb_tier_desc_t()
    t.host_weights = kw.pop("host_weights", 0x50000000)
    t.host_accum = kw.pop("host_accum", 0x60000000)
    t.cache_rows = kw.pop("cache_rows", 4 * eb.EMB_CACHE_WAYS)
    t.cache_state = kw.pop("cache_state", 0x70000000)
    assert not kw
    return t


@pytest.mark.parametrize("dkw,tkw,code", [
    (dict(init_storage=1), dict(host_weights=0x50000008), eb.EMB_ERR_INVALID_ARG),
    (dict(init_storage=1, hashed=1, hash_capacity=1024, hash_slots=0x40000000), dict(),
     eb.EMB_ERR_UNSUPPORTED),
    (dict(init_storage=1), dict(cache_rows=0), eb.EMB_ERR_INVALID_ARG),
    (dict(init_storage=1), dict(cache_rows=3 * eb.EMB_CACHE_WAYS), eb.EMB_ERR_INVALID_ARG),
    (dict(init_storage=1), dict(cache_rows=32 * eb.EMB_CACHE_WAYS), eb.EMB_ERR_INVALID_ARG),
    (dict(init_storage=1), dict(host_weights=None), eb.EMB_ERR_INVALID_ARG),
    (dict(init_storage=1), dict(host_accum=0x60000008), eb.EMB_ERR_INVALID_ARG),
    (dict(init_storage=1), dict(cache_state=0x70000010), eb.EMB_ERR_INVALID_ARG),
    (dict(init_storage=1, dim=6), dict(), eb.EMB_ERR_INVALID_ARG),
])
def test_create_tiered_rejects(dkw, tkw, code):
    # rows [100, 200]: 300 rows in all, so 32 sets of 16 do not fit
    d, _keep = _desc(**dkw)
    st, h = eb.emb_table_create_tiered(d, _tier(**tkw), 0)
    assert st == code and h is None


def test_cache_calls_on_a_dense_handle():
    d, _keep = _desc(rows=[1000], dim=16)
    st, h = eb.emb_table_create(d, 0)
    assert st == eb.EMB_OK and h
    try:
        assert eb.emb_cache_flush(h, 0) == eb.EMB_ERR_UNSUPPORTED
        assert eb.emb_cache_prepare(h, 4, 4, 0x50000000, 1 << 20, 0) == eb.EMB_ERR_UNSUPPORTED
        assert eb.emb_cache_stats(h, 0)[0] == eb.EMB_ERR_UNSUPPORTED
    finally:
        eb.emb_table_destroy(h)
    assert eb.emb_cache_flush(None, 0) == eb.EMB_ERR_INVALID_ARG
    assert eb.emb_status_string(eb.EMB_ERR_CACHE_FULL) == "cache set full"


def test_decay_backward_host_checks():
    d, _keep = _desc(rows=[1000, 24], dim=64)
    st, h = eb.emb_table_create(d, 0)
    assert st == eb.EMB_OK and h
    try:
        ws = eb.emb_workspace_bytes(h, 4096, 10000)
        fake, per = 0x50000000, 0x60000000
        call = lambda rho=0.9, periods=per, w=fake, wsb=ws, grad=fake: \
            eb.emb_bag_backward_adagrad_decay_prepared(h, 4096, 10000, 0, grad, 0.01, 1e-8, rho,
                                                       3, periods, w, wsb, 0)
        for bad in (0.0, -0.5, 1.5, float("nan"), float("inf")):
            assert call(rho=bad) == eb.EMB_ERR_INVALID_ARG, bad
        assert call(periods=None) == eb.EMB_ERR_INVALID_ARG
        assert call(periods=per + 2) == eb.EMB_ERR_INVALID_ARG  # 4-byte alignment
        assert call(grad=None) == eb.EMB_ERR_INVALID_ARG
        assert call(wsb=ws - 1) == eb.EMB_ERR_WORKSPACE
        assert eb.emb_bag_backward_adagrad_decay_prepared(h, 0, 0, 0, fake, 0.01, 1e-8, 1.0, 0,
                                                          per, fake, ws, 0) == eb.EMB_OK
    finally:
        eb.emb_table_destroy(h)


def test_evict_host_checks():
    d, _keep = _desc(rows=[1000], dim=16)
    st, h = eb.emb_table_create(d, 0)
    assert st == eb.EMB_OK
    try:  # a dense table has no keys to evict
        assert eb.emb_hash_evict_workspace_bytes(h) == 0
        assert eb.emb_hash_evict(h, 0x50000000, 3, None, 0x60000000, 1 << 30,
                                 0) == eb.EMB_ERR_UNSUPPORTED
    finally:
        eb.emb_table_destroy(h)
    for free_rows, expect in ((None, eb.EMB_ERR_UNSUPPORTED), (0x48000000, None)):
        d, _keep = _desc(rows=[600, 100], dim=16, hashed=1, hash_capacity=1024,
                         hash_slots=0x40000000, free_rows=free_rows)
        st, h = eb.emb_table_create(d, 0)
        assert st == eb.EMB_OK
        try:
            ws = eb.emb_hash_evict_workspace_bytes(h)
            assert ws >= 2 * 1024 * 16 + 700 and ws % 256 == 0
            call = lambda lu=0x50000000, kc=None, w=0x60000000, n=ws: eb.emb_hash_evict(
                h, lu, 3, kc, w, n, 0)
            if expect is not None:
                assert call() == expect
                continue
            assert call(lu=None) == eb.EMB_ERR_INVALID_ARG
            assert call(lu=0x50000002) == eb.EMB_ERR_INVALID_ARG
            assert call(kc=0x58000001) == eb.EMB_ERR_INVALID_ARG
            assert call(n=ws - 1) == eb.EMB_ERR_WORKSPACE
            assert call(w=0x60000010) == eb.EMB_ERR_WORKSPACE
        finally:
            eb.emb_table_destroy(h)
    d, _keep = _desc(rows=[600], dim=16, hashed=1, hash_capacity=1024, hash_slots=0x40000000,
                     free_rows=0x48000002)  # misaligned queue
    assert eb.emb_table_create(d, 0)[0] == eb.EMB_ERR_INVALID_ARG


def test_interaction_host_checks():
    d, _keep = _desc(rows=[100, 200, 50], dim=32)
    st, h = eb.emb_table_create(d, 0)
    assert st == eb.EMB_OK
    try:
        assert eb.emb_interact_out_dim(h) == 32 + 4 * 3 // 2
        fake = 0x50000000
        f = lambda dense=fake, pool=0, out=fake, batch=64: eb.emb_bag_forward_interact(
            h, fake, fake, batch, 100, pool, dense, out, 0)
        assert f(dense=None) == eb.EMB_ERR_INVALID_ARG
        assert f(dense=fake + 4) == eb.EMB_ERR_INVALID_ARG  # 16-byte alignment
        assert f(pool=5) == eb.EMB_ERR_INVALID_ARG
        assert f(out=None) == eb.EMB_ERR_INVALID_ARG
        assert f(batch=0) == eb.EMB_OK
        assert eb.emb_interact_backward(h, fake, fake, 64, 100, 0, fake, None, fake, fake,
                                        0) == eb.EMB_ERR_INVALID_ARG
        assert eb.emb_interact_backward(h, fake, fake, 0, 0, 0, fake, fake, fake, fake,
                                        0) == eb.EMB_OK
    finally:
        eb.emb_table_destroy(h)
    for rows, dim in (([10] * 32, 16), ([10, 10], 20), ([10, 10], 272)):
        d, _keep = _desc(rows=rows, dim=dim)
        st, h = eb.emb_table_create(d, 0)
        assert st == eb.EMB_OK
        try:  # T + 1 > 32, D % 16 != 0, D > 256
            assert eb.emb_bag_forward_interact(h, 0x50000000, 0x50000000, 4, 8, 0, 0x50000000,
                                               0x50000000, 0) == eb.EMB_ERR_UNSUPPORTED
        finally:
            eb.emb_table_destroy(h)


def test_int8_payload_host_checks():
    # argument checks only: nothing is launched
    x, c, s, y = 0x50000000, 0x50000000, 0x50000000, 0x50000000
    def q(*a):
        return eb.emb_quantize_rows_int8(*a, 0)

    def dq(*a):
        return eb.emb_dequantize_rows_int8(*a, 0)

    assert q(x, 0, 128, c, s) == eb.EMB_OK and dq(c, s, 0, 128, y) == eb.EMB_OK
    for dim in (0, 2, 6, 1028):  # a multiple of 4 in [4, 1024]
        assert q(x, 4, dim, c, s) == eb.EMB_ERR_INVALID_ARG
        assert dq(c, s, 4, dim, y) == eb.EMB_ERR_INVALID_ARG
    assert q(x, -1, 8, c, s) == eb.EMB_ERR_INVALID_ARG
    assert q(None, 4, 8, c, s) == eb.EMB_ERR_INVALID_ARG
    assert q(x + 4, 4, 8, c, s) == eb.EMB_ERR_INVALID_ARG  # x 16-byte aligned
    assert q(x, 4, 8, c + 2, s) == eb.EMB_ERR_INVALID_ARG  # codes 4-byte aligned
    assert q(x, 4, 8, c, s + 1) == eb.EMB_ERR_INVALID_ARG
    assert dq(c, s, 4, 8, y + 8) == eb.EMB_ERR_INVALID_ARG  # y 16-byte aligned
    assert dq(c, None, 4, 8, y) == eb.EMB_ERR_INVALID_ARG
