"""Seeded synthetic inputs for the sparse embedding layer.

This module only draws random inputs (table sizes, CSR bags, ids, raw keys,
upstream gradients).  It holds none of the layer's arithmetic and is the one
piece shared by the GPU path's tests and benchmark and by the CPU oracle's
tests: both receive the same arrays as data.

The five workloads follow the shapes the pages describe for DLRM-style
training (26 categorical tables and global batch 65536 with Adagrad in the
synthetic-model benchmarks of the "NVIDIA Merlin Distributed Embeddings" page,
section "Performance"; multi-hot feature fields and hash-identified raw keys
in the "Merlin HugeCTR interview" page, section two).  The pages benchmark on
the Criteo 1TB click logs and MLPerf DLRM; those datasets are not used: seeded
Zipf-distributed ids over log-uniform table sizes stand in for them.

Random streams: numpy default_rng(SeedSequence([seed, cfg, stream, t, batch]))
with stream 0 = table sizes, 1 = ids or keys, 2 = bag lengths, 3 = upstream
gradient, 4 = key universe.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

S_ROWS, S_IDS, S_LENS, S_GRAD, S_UNIVERSE, S_PREFILL = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass
class Workload:
    name: str
    cfg: int
    T: int
    D: int
    B: int
    rows: np.ndarray            # rows (capacity) per table, int64 [T]
    pool_mean: bool
    bag: tuple                  # ("fixed", L) or ("poisson", mean, lo, hi)
    ids: tuple                  # ("uniform",) or ("zipf", alpha)
    hashed: bool = False
    hash_capacity: int = 0      # slots per table (power of two)
    max_load: float = 0.625
    universe: int = 0           # distinct raw keys per table
    init_lo: float = -0.05
    init_hi: float = 0.05
    init_std: float = 0.01
    accum_init: float = 0.1
    lr: float = 0.01
    eps: float = 1e-8
    seed: int = 1234

    @property
    def bags(self) -> int:
        return self.T * self.B

    @property
    def total_rows(self) -> int:
        return int(self.rows.sum())

    def describe(self) -> dict:
        return {
            "workload": self.name, "tables": self.T, "dim": self.D, "batch": self.B,
            "rows_total": self.total_rows, "pool": "mean" if self.pool_mean else "sum",
            "bag": list(self.bag), "ids": list(self.ids), "hashed": self.hashed,
        }


def _rng(seed: int, cfg: int, stream: int, t: int = 0, batch: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, stream, t, batch]))


def log_uniform_rows(T: int, lo_exp: float, hi_exp: float, seed: int, cfg: int) -> np.ndarray:
    """N_t = round(10**U(lo_exp, hi_exp)), one draw per table."""
    e = _rng(seed, cfg, S_ROWS).uniform(lo_exp, hi_exp, size=T)
    return np.rint(10.0 ** e).astype(np.int64)


def workload(cfg: int, seed: int = 1234, **over) -> Workload:
    """The five workloads at full size; keyword overrides shrink them for tests."""
    if cfg == 1:
        w = Workload("single-table 10000x16, B=256, L=4, uniform ids, sum", 1, T=1, D=16, B=256,
                     rows=np.array([10_000], np.int64), pool_mean=False, bag=("fixed", 4),
                     ids=("uniform",), seed=seed)
    elif cfg == 2:
        T = over.pop("T", 26)
        rows = over.pop("rows", None)
        if rows is None:
            rows = log_uniform_rows(T, 2.0, 7.0, seed, 2)
        w = Workload("26 one-hot tables, rows log-uniform 1e2..1e7, D=128, B=65536, "
                     "Zipf(1.05), sum", 2, T=T, D=128, B=65536, rows=np.asarray(rows, np.int64),
                     pool_mean=False, bag=("fixed", 1), ids=("zipf", 1.05), seed=seed)
    elif cfg == 3:
        T = over.pop("T", 8)
        w = Workload("multi-hot 8x5e6 rows, D=64, B=16384, L~Poisson(20) in [1,100], "
                     "Zipf(1.2), mean", 3, T=T, D=64, B=16384,
                     rows=np.full(T, 5_000_000, np.int64), pool_mean=True,
                     bag=("poisson", 20.0, 1, 100), ids=("zipf", 1.2), seed=seed)
    elif cfg == 4:
        T = over.pop("T", 2)
        w = Workload("capacity 2x5e7 rows, D=256, B=65536, uniform ids, sum", 4, T=T, D=256,
                     B=65536, rows=np.full(T, 50_000_000, np.int64), pool_mean=False,
                     bag=("fixed", 1), ids=("uniform",), seed=seed)
    elif cfg == 5:
        T = over.pop("T", 4)
        cap = over.pop("hash_capacity", 1 << 25)
        max_load = over.pop("max_load", 0.625)
        w = Workload("hashed 4 tables, 2^25 slots, 2e7-key universe, Zipf(1.1), D=64, B=32768, "
                     "L=8, sum", 5, T=T, D=64, B=32768,
                     rows=np.full(T, int(math.floor(max_load * cap)), np.int64), pool_mean=False,
                     bag=("fixed", 8), ids=("zipf", 1.1), hashed=True, hash_capacity=cap,
                     max_load=max_load, universe=20_000_000, seed=seed)
    else:
        raise ValueError(f"unknown workload {cfg}")
    for k, v in over.items():
        if not hasattr(w, k):
            raise TypeError(f"unknown workload field {k}")
        if k == "rows":
            v = np.asarray(v, np.int64)
        setattr(w, k, v)
    if over:
        w.name = w.name + " (scaled: " + ", ".join(f"{k}={over[k] if k != 'rows' else '...'}"
                                                   for k in sorted(over)) + ")"
    return w


# ---------------------------------------------------------------- bags / ids

def bag_lengths(w: Workload, batch: int = 0) -> np.ndarray:
    """Bag lengths in table-major order (bag b = t*B + s), int64 [T*B]."""
    kind = w.bag[0]
    if kind == "fixed":
        return np.full(w.bags, int(w.bag[1]), np.int64)
    if kind == "poisson":
        lam, lo, hi = w.bag[1], w.bag[2], w.bag[3]
        out = np.empty(w.bags, np.int64)
        for t in range(w.T):
            r = _rng(w.seed, w.cfg, S_LENS, t, batch)
            out[t * w.B:(t + 1) * w.B] = np.clip(r.poisson(lam, size=w.B), lo, hi)
        return out
    raise ValueError(kind)


def offsets_from_lengths(lengths: np.ndarray) -> np.ndarray:
    off = np.zeros(lengths.size + 1, np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


_ZIPF_CDF: dict = {}


def zipf_cdf(n: int, alpha: float) -> np.ndarray:
    """CDF of the Zipf law truncated to ranks 1..n: P(rank = k) ~ k**-alpha."""
    key = (int(n), float(alpha))
    c = _ZIPF_CDF.get(key)
    if c is None:
        p = np.arange(1, n + 1, dtype=np.float64) ** (-alpha)
        c = np.cumsum(p)
        c /= c[-1]
        if len(_ZIPF_CDF) > 8:
            _ZIPF_CDF.clear()
        _ZIPF_CDF[key] = c
    return c


def zipf_ranks(rng: np.random.Generator, n: int, alpha: float, size: int) -> np.ndarray:
    """Zero-based ranks (rank 1 -> 0) by inverse-CDF sampling."""
    c = zipf_cdf(n, alpha)
    r = np.searchsorted(c, rng.random(size), side="right")
    return np.minimum(r, n - 1).astype(np.int64)


def gen_batch(w: Workload, batch: int = 0):
    """CSR offsets [T*B+1] and per-occurrence table-local ids [nnz] (int64).

    For hashed workloads the ids are ranks into the table's key universe; use
    gen_keys to turn them into raw 64-bit keys.
    """
    lens = bag_lengths(w, batch)
    offsets = offsets_from_lengths(lens)
    ids = np.empty(int(offsets[-1]), np.int64)
    space = w.universe if w.hashed else None
    for t in range(w.T):
        a, b = int(offsets[t * w.B]), int(offsets[(t + 1) * w.B])
        n = int(space if space is not None else w.rows[t])
        r = _rng(w.seed, w.cfg, S_IDS, t, batch)
        if w.ids[0] == "uniform":
            ids[a:b] = r.integers(0, n, size=b - a, dtype=np.int64)
        else:
            ids[a:b] = zipf_ranks(r, n, w.ids[1], b - a)
    return offsets, ids


_UNIVERSE: dict = {}


def key_universe(w: Workload, t: int) -> np.ndarray:
    """w.universe distinct uint64 keys for table t (never the all-ones value)."""
    k = (w.seed, w.cfg, t, w.universe)
    u = _UNIVERSE.get(k)
    if u is not None:
        return u
    r = _rng(w.seed, w.cfg, S_UNIVERSE, t)
    top = np.uint64(0xFFFFFFFFFFFFFFFF)
    keys = r.integers(0, top, size=w.universe, dtype=np.uint64)  # top excluded
    while True:
        uniq, first = np.unique(keys, return_index=True)
        if uniq.size == keys.size:
            break
        keep = np.zeros(keys.size, bool)
        keep[first] = True
        extra = r.integers(0, top, size=int((~keep).sum()), dtype=np.uint64)
        keys = np.concatenate([keys[keep], extra])
    if len(_UNIVERSE) > 8:
        _UNIVERSE.clear()
    _UNIVERSE[k] = keys
    return keys


def gen_keys(w: Workload, offsets: np.ndarray, ranks: np.ndarray) -> np.ndarray:
    """Raw keys of a hashed workload: key = universe_t[rank]."""
    keys = np.empty(ranks.size, np.uint64)
    for t in range(w.T):
        a, b = int(offsets[t * w.B]), int(offsets[(t + 1) * w.B])
        keys[a:b] = key_universe(w, t)[ranks[a:b]]
    return keys


def prefill_keys(w: Workload, t: int, n: int) -> np.ndarray:
    """Keys of ranks 0 .. n-1 of table t in a seeded random order: the keys a
    long training run has already inserted (warm start of a hashed workload)."""
    r = _rng(w.seed, w.cfg, S_PREFILL, t)
    return key_universe(w, t)[r.permutation(n)]


def gen_grad(w: Workload, batch: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Upstream gradient N(0, 1), float32 [B, T, D]."""
    r = _rng(w.seed, w.cfg, S_GRAD, 0, batch)
    if out is None:
        out = np.empty((w.B, w.T, w.D), np.float32)
    r.standard_normal(out=out.reshape(-1), dtype=np.float32)
    return out


def random_small(seed: int, T: int, D: int, B: int, rows, max_len: int = 5,
                 empty_frac: float = 0.0):
    """Tiny CSR batch with duplicates, ragged bags and optional empty bags."""
    r = np.random.default_rng(seed)
    rows = np.asarray(rows, np.int64)
    lens = r.integers(1, max_len + 1, size=T * B)
    if empty_frac > 0:
        lens[r.random(T * B) < empty_frac] = 0
    offsets = offsets_from_lengths(lens.astype(np.int64))
    ids = np.empty(int(offsets[-1]), np.int64)
    for t in range(T):
        a, b = int(offsets[t * B]), int(offsets[(t + 1) * B])
        ids[a:b] = r.integers(0, rows[t], size=b - a)
    grad = r.standard_normal((B, T, D)).astype(np.float32)
    return offsets, ids, grad
