"""The GPU hash table against the oracle at the loads the benchmark runs at and
beyond, through the C ABI: ids and the key<->row map bit-exact over many calls
at 0.566, 0.625 and 0.9 of the slots (the largest load a table may be created
with), calls whose new keys exceed the free rows on small tables (all or
nothing), admission whose counted keys would overfill the slot array (the
slot bound), and offsets that are not valid (the table is left as it was).

Every table here is checked through `check_hash_state`: live-row counters,
the exported key of every row against the oracle's std::map, and the rows'
initial values.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from tests.test_gpu_parity import _hash_call, _t, check_hash_state, make_pair, status

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from recommender_embedding_tables_amd import embtab as eb  # noqa: E402

DEV = torch.device("cuda")
SLOT_LOAD = 0.9  # share of a table's slots that may hold keys (live or counted)


def _keys(rng, n):
    """n distinct random 64-bit keys, none of them the reserved all-ones key."""
    k = np.unique(rng.integers(1, np.iinfo(np.int64).max, int(n * 1.1) + 16, dtype=np.int64))
    rng.shuffle(k)
    assert k.size >= n
    return k[:n].astype(np.uint64)


def _batch(rng, pools, per_table, B):
    """One call: T tables, each drawing per_table occurrences from its pool
    with repeats (heavy duplicates), in B bags of ragged length."""
    T = len(pools)
    keys, lens = [], []
    for t in range(T):
        p = pools[t]
        # a skewed draw: half the occurrences from the first 1/16 of the pool
        hot = rng.integers(0, max(1, p.size // 16), per_table // 2)
        cold = rng.integers(0, p.size, per_table - per_table // 2)
        sel = np.concatenate([hot, cold])
        rng.shuffle(sel)
        keys.append(p[sel])
        cut = np.sort(rng.integers(0, per_table + 1, B - 1))
        lens.append(np.diff(np.concatenate([[0], cut, [per_table]])))
    offsets = np.concatenate([[0], np.cumsum(np.concatenate(lens))]).astype(np.int64)
    return offsets, np.concatenate(keys)


def _admit(tabs, counts, offsets, keys, B, N):
    ids = torch.empty(keys.size, dtype=torch.int64, device=DEV)
    ws, need = tabs.workspace(B, keys.size)
    eb.check(eb.emb_hash_find_or_insert_admit(tabs.handle, _t(offsets), _t(keys.view(np.int64)),
                                              B, keys.size, ids, N, counts, ws, need),
             "find_or_insert_admit")
    torch.cuda.synchronize()
    return ids.cpu().numpy()


@pytest.mark.parametrize("load,cap", [(0.566, 1 << 16), (0.625, 1 << 16), (0.9, 1 << 15),
                                      (0.625, 1 << 18)])
def test_hash_parity_up_to_load(load, cap):
    """Fill two tables call by call to `load` of their slots (rows =
    floor(load * cap)), every call a mix of known and new keys with heavy
    duplicates; ids bit-exact each call, the key<->row map at the end."""
    T, B = 2, 512
    rows = np.full(T, int(load * cap), np.int64)
    tabs, o = make_pair(rows, 16, seed=31, hashed=True, cap=cap, max_load=max(load, 0.566))
    rng = np.random.default_rng(int(load * 1000) + cap)
    universe = [_keys(rng, int(rows[t])) for t in range(T)]
    inserted = 0
    calls = 0
    while inserted < rows[0]:
        grow = min(int(rows[0]) - inserted, max(cap // 8, 1))
        pools = [u[:inserted + grow] for u in universe]
        offsets, keys = _batch(rng, pools, 3 * grow, B)
        ids = _hash_call(tabs, offsets, keys, B)
        ref, fl = o.find_or_insert(offsets, keys, B)
        assert fl == 0
        np.testing.assert_array_equal(ids, ref)
        assert status(tabs) == (eb.EMB_OK, 0)
        inserted = min(o.n_live(t) for t in range(T))
        calls += 1
        if calls > 64:
            break
    # the draws reach every key of the pool by the end: top the tables up
    for t in range(T):
        missing = np.setdiff1d(universe[t], o.export(t)[0])
        if missing.size:
            offsets = np.zeros(T * B + 1, np.int64)
            offsets[(t * B + 1):] = missing.size
            kk = missing.astype(np.uint64)
            ids = _hash_call(tabs, offsets, kk, B)
            ref, fl = o.find_or_insert(offsets, kk, B)
            assert fl == 0
            np.testing.assert_array_equal(ids, ref)
    assert all(o.n_live(t) == rows[t] for t in range(T))
    # at full load: repeated lookups of everything, with duplicates
    for _ in range(2):
        offsets, keys = _batch(rng, universe, 4096, B)
        ids = _hash_call(tabs, offsets, keys, B)
        ref, fl = o.find_or_insert(offsets, keys, B)
        assert fl == 0
        np.testing.assert_array_equal(ids, ref)
    assert status(tabs) == (eb.EMB_OK, 0)
    check_hash_state(tabs, o)


@pytest.mark.parametrize("cap", [64, 4096])
def test_hash_call_beyond_free_rows_is_undone(cap):
    """Small tables: calls insert until one call's distinct new keys exceed the
    rows left; that call inserts nothing (FULL), the table is exactly as
    before, and the next call that fits goes through."""
    T, B = 2, 8
    rows = np.full(T, int(SLOT_LOAD * cap), np.int64)
    tabs, o = make_pair(rows, 8, seed=41, hashed=True, cap=cap, max_load=SLOT_LOAD)
    rng = np.random.default_rng(cap)
    fresh = [_keys(rng, 3 * cap) for _ in range(T)]
    used = [0] * T
    saw_full = False
    for call in range(12):
        # table 0 gets about a third of its rows each call, table 1 a few
        n0 = max(2, int(rows[0]) // 3 + int(rng.integers(0, 3)))
        pools = [fresh[0][:used[0] + n0], fresh[1][:used[1] + 2]]
        offsets, keys = _batch(rng, pools, 2 * n0 + 8, B)
        before = [o.export(t) for t in range(T)]
        ids = _hash_call(tabs, offsets, keys, B)
        ref, fl = o.find_or_insert(offsets, keys, B)
        np.testing.assert_array_equal(ids, ref)
        st, flags = status(tabs)
        if fl & orc.ERR_TABLE_FULL:
            saw_full = True
            assert st == eb.EMB_ERR_TABLE_FULL and flags == eb.EMB_FLAG_TABLE_FULL
            for t in range(T):  # nothing changed
                k, r = o.export(t)
                np.testing.assert_array_equal(k, before[t][0])
                np.testing.assert_array_equal(r, before[t][1])
            check_hash_state(tabs, o)
            # a call that fits afterwards: keys already in the table, one new
            k0 = np.concatenate([o.export(0)[0][:3], fresh[0][used[0]:used[0] + 1]])
            offs = np.zeros(T * B + 1, np.int64)
            offs[1:] = k0.size
            ids = _hash_call(tabs, offs, k0, B)
            ref, fl = o.find_or_insert(offs, k0, B)
            assert fl == 0 or fl == orc.ERR_TABLE_FULL
            np.testing.assert_array_equal(ids, ref)
            status(tabs)
            break
        assert st == eb.EMB_OK
        used = [o.n_live(t) for t in range(T)]
    assert saw_full
    check_hash_state(tabs, o)


def test_admission_slot_bound_keeps_probes_short():
    """Admission on a 64-slot table with 8 rows: keys seen once stay counted
    and hold slots.  Once the counted and live keys would pass 0.9 of the
    slots, a call keeps none of its unknown keys (FULL, ids -1), the counted
    keys' counts still advance, and later calls go on; every call matches the
    oracle run with the same slot bound."""
    cap, N = 64, 3
    limit = int(SLOT_LOAD * cap)
    rows = np.array([8], np.int64)
    tabs = eb.EmbTables(rows, 8, hashed=True, hash_capacity=cap, max_load=0.125, seed=3)
    o = orc.Oracle(rows, 8, hashed=True, seed=3, slot_limit=limit)
    counts = torch.zeros(cap, dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(17)
    universe = _keys(rng, 400)
    B, nxt, saw_full, saw_row = 4, 0, False, False
    for call in range(30):
        # a few keys seen before (they may reach N) and a burst of new ones
        old = universe[rng.integers(0, max(nxt, 1), 6)] if nxt else universe[:0]
        new = universe[nxt:nxt + int(rng.integers(3, 9))]
        nxt += new.size
        keys = np.concatenate([old, new, old[:2]]).astype(np.uint64)
        offsets = np.array([0, 3, 6, 9, keys.size], np.int64)
        offsets = np.minimum(offsets, keys.size)
        ids = _admit(tabs, counts, offsets, keys, B, N)
        ref, fl = o.find_or_insert_admit(offsets, keys, B, N)
        np.testing.assert_array_equal(ids, ref, err_msg=f"call {call}")
        st, flags = status(tabs)
        if fl & orc.ERR_TABLE_FULL:
            saw_full = True
            assert st == eb.EMB_ERR_TABLE_FULL
        else:
            assert st == eb.EMB_OK
        saw_row = saw_row or bool((ids >= 0).any())
    assert saw_full and saw_row
    check_hash_state(tabs, o)


@pytest.mark.parametrize("admission", [False, True])
def test_hash_bad_offsets_change_nothing(admission):
    """Offsets that do not start at 0, do not end at nnz, or fall inside a
    table: the call is flagged BAD_OFFSETS and inserts nothing (the oracle
    refuses it outright); admission counts do not advance either, which the
    calls after it show."""
    T, B, cap = 2, 3, 256
    rows = np.full(T, 100, np.int64)
    tabs, o = make_pair(rows, 8, seed=9, hashed=True, cap=cap)
    counts = torch.zeros(T * cap, dtype=torch.int32, device=DEV) if admission else None
    N = 2

    def call(offsets, keys):
        if admission:
            return _admit(tabs, counts, offsets, keys, B, N), \
                o.find_or_insert_admit(offsets, keys, B, N)
        return _hash_call(tabs, offsets, keys, B), o.find_or_insert(offsets, keys, B)

    good = np.array([0, 2, 4, 6, 8, 9, 12], np.int64)
    keys = np.array([11, 12, 13, 11, 14, 15, 21, 22, 23, 21, 24, 25], np.uint64)
    ids, (ref, fl) = call(good, keys)
    np.testing.assert_array_equal(ids, ref)
    assert status(tabs) == (eb.EMB_OK, 0)
    fresh = np.array([31, 32, 33, 31, 34, 35, 41, 42, 43, 41, 44, 45], np.uint64)
    bad_cases = [
        np.array([1, 2, 4, 6, 8, 9, 12], np.int64),   # does not start at 0
        np.array([0, 2, 4, 6, 8, 9, 11], np.int64),   # does not end at nnz
        np.array([0, 5, 3, 6, 8, 9, 12], np.int64),   # falls inside table 0
        np.array([0, 2, 4, 13, 8, 9, 12], np.int64),  # table 1 starts past the end
    ]
    before = [o.export(t) for t in range(T)]
    for bad in bad_cases:
        ids, (ref, fl) = call(bad, fresh)
        assert fl == orc.ERR_BAD_OFFSETS  # the oracle refuses the call
        st, flags = status(tabs)
        assert st == eb.EMB_ERR_BAD_OFFSETS and flags == eb.EMB_FLAG_BAD_OFFSETS
        assert ((ids == -1) | (ids >= 0)).all()
        check_hash_state(tabs, o)
        for t in range(T):
            np.testing.assert_array_equal(o.export(t)[0], before[t][0])
    # the same keys with good offsets now: counts start from where they were
    for _ in range(2):
        ids, (ref, fl) = call(good, fresh)
        np.testing.assert_array_equal(ids, ref)
        assert status(tabs) == (eb.EMB_OK, 0)
    check_hash_state(tabs, o)
