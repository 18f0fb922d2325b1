"""Host-side rules of bench.py, on the CPU: the options it refuses before any
GPU work, and the algorithmic byte counts its roofline divides by, checked
against the sizes the workloads fix (output [B, T, D] fp32 written once,
distinct rows read once, 16 bytes of W and G read and written per element of
each touched row)."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

from recommender_embedding_tables_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


@pytest.mark.skipif(not os.path.exists(os.path.join(ROOT, "recommender_embedding_tables_amd",
                                                    "libembtab.so")),
                    reason="the HIP library is not built")
def test_schedules_that_do_not_fit_the_workload_are_refused():
    r = _run("--workload", "1", "--schedule", "pipelined4")
    assert r.returncode == 2 and "hashed tables" in r.stderr
    r = _run("--workload", "1", "--graph")  # default schedule is pipelined
    assert r.returncode == 2 and "--graph" in r.stderr
    r = _run("--workload", "1", "--evict-every", "4", "--schedule", "prepared")
    assert r.returncode == 2 and "hashed workload" in r.stderr


def test_algorithmic_bytes_of_the_26_table_step():
    bench = _bench_module()
    w = synth.workload(2)
    offsets, ids = synth.gen_batch(w, 0)
    nnz, bags = ids.size, w.T * w.B
    assert nnz == bags == 1_703_936  # one-hot
    U = 300_000
    b = bench.algorithmic_bytes(w, offsets, ids, U)
    out_bytes = 65536 * 26 * 128 * 4
    assert out_bytes == 872_415_232
    csr = (bags + 1) * 8 + nnz * 8
    # forward: CSR in, each distinct row read once, the output written once
    assert b["forward"] == csr + U * 128 * 4 + out_bytes
    # reduction + Adagrad: a sorted key and grad-row index per occurrence, the
    # upstream gradient read once, W and G read and written for U rows
    assert b["reduce_adagrad"] == nnz * 8 + out_bytes + U * 128 * 16
    assert b["step"] == sum(v for k, v in b.items() if k != "step")
    assert "hash" not in b


def test_mean_pooling_adds_the_scale_per_occurrence():
    bench = _bench_module()
    w = synth.workload(3, T=2, B=1000)
    offsets, ids = synth.gen_batch(w, 0)
    b = bench.algorithmic_bytes(w, offsets, ids, 500)
    dense = w.B * w.T * w.D * 4
    assert b["reduce_adagrad"] == ids.size * 12 + dense + 500 * w.D * 16


def test_hashed_step_counts_the_key_and_slot_traffic():
    bench = _bench_module()
    w = synth.workload(5, T=2, B=1000)
    offsets, ids = synth.gen_batch(w, 0)
    U = 4000
    b = bench.algorithmic_bytes(w, offsets, ids, U)
    # offsets in, u64 keys in, one 16-byte slot per distinct key, int64 ids out
    assert b["hash"] == (w.T * w.B + 1) * 8 + ids.size * 8 + U * 16 + ids.size * 8
    assert np.isclose(b["step"], sum(v for k, v in b.items() if k != "step"))


def test_table_wise_shards_cover_every_table_once_and_balance_lookups():
    bench = _bench_module()
    w = synth.workload(2)
    for P in (2, 4, 8, 26):
        sh = bench.shard_tables(w.rows, P)
        assert len(sh) == P
        assert sorted(np.concatenate(sh).tolist()) == list(range(w.T))
        sizes = [len(s) for s in sh]
        assert max(sizes) - min(sizes) <= 1  # one-hot lookups per GPU differ by one table
        assert all(np.all(np.diff(s) > 0) for s in sh)
    # the snake order gives the largest table's owner none of the next P - 1 largest
    sh = bench.shard_tables(w.rows, 8)
    order = np.argsort(-w.rows, kind="stable")
    owner = {int(t): r for r, s in enumerate(sh) for t in s}
    assert len({owner[int(t)] for t in order[:8]}) == 8


@pytest.mark.skipif(not os.path.exists(os.path.join(ROOT, "recommender_embedding_tables_amd",
                                                    "libembtab.so")),
                    reason="the HIP library is not built")
def test_shard_option_is_refused_where_it_does_not_apply():
    r = _run("--workload", "5", "--shard", "0/4")
    assert r.returncode == 2 and "--shard" in r.stderr
    r = _run("--shard", "8/8")
    assert r.returncode == 2 and "--shard" in r.stderr


@pytest.mark.skipif(not os.path.exists(os.path.join(ROOT, "recommender_embedding_tables_amd",
                                                    "libembtab.so")),
                    reason="the HIP library is not built")
def test_int8_exchange_needs_the_pooled_output():
    r = _run("--interact", "--schedule", "prepared", "--int8-exchange")
    assert r.returncode == 2 and "--int8-exchange" in r.stderr


def test_stored_traffic_is_dropped_once_the_kernel_sources_change(tmp_path, monkeypatch):
    # The committed counter summaries count only for the kernel sources they
    # were taken from: a copy of the reduction's summary with another source
    # hash gives no traffic, and then no step ratio for the gate either.
    bench = _bench_module()
    assert bench.stored_traffic("reduce_adagrad", 3) is None  # the 26-table workload only
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = open(os.path.join(ROOT, "profiles", "reduce_adagrad_26tables_traffic.txt")).read()
    lines = [("source_sha256: " + "0" * 64) if ln.startswith("source_sha256:") else ln
             for ln in src.splitlines()]
    (prof / "reduce_adagrad_26tables_traffic.txt").write_text("\n".join(lines) + "\n")
    (prof / "step_26tables_traffic.txt").write_text("measured_over_algorithmic: 1.0\n")
    for f in [ln.split(":", 1)[1].split() for ln in lines if ln.startswith("source_files:")][0]:
        (tmp_path / f).parent.mkdir(parents=True, exist_ok=True)
        (tmp_path / f).write_bytes(open(os.path.join(ROOT, f), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("reduce_adagrad", 2) is None
    assert bench.stored_step_traffic_ratio() is None
    # with the matching hash the same copy gives the stored figures
    (prof / "reduce_adagrad_26tables_traffic.txt").write_text(src)
    assert bench.stored_traffic("reduce_adagrad", 2) > 0
    assert bench.stored_step_traffic_ratio() == 1.0
