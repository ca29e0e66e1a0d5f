"""bench.py's host-side contract (CPU only): the one-GPU guard, the rocprofv3 database
readers behind the profiler summaries, the traffic lookup's source-hash gate, and the
CPU oracle baseline on a tiny workload."""

from __future__ import annotations

import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _rocpd(path, kernels=(), counters=()):
    """A minimal database with the two tables the readers use."""
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, start integer, end integer)")
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into kernels values (?, ?, ?)", kernels)
    con.executemany("insert into counters_collection values (?, ?, ?)", counters)
    con.commit()
    con.close()


def test_trace_durations_and_counter_means(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    _rocpd(str(d / "a_results.db"), kernels=[("void qgemv::k(x)", 0, 4000), ("void qgemv::k(x)", 10, 2010),
                                             ("copy", 0, 500)],
           counters=[("void qgemv::k(x)", "FETCH_SIZE", 10.0), ("void qgemv::k(x)", "FETCH_SIZE", 14.0)])
    dur = bench.trace_durations(str(d))
    assert sorted(dur["void qgemv::k(x)"]) == [2000, 4000] and dur["copy"] == [500]
    cm = bench.counter_means(str(d))
    assert cm["void qgemv::k(x)"]["FETCH_SIZE"] == (12.0, 2)


def test_trace_summary_means_the_last_launches(tmp_path, capsys):
    """Durations come back in launch order, across databases, and the summary's last-K
    column averages the kernel's last K launches (a profiled run's timed calls)."""
    d = tmp_path / "run"
    d.mkdir()
    _rocpd(str(d / "a_results.db"), kernels=[("k", 300, 1300), ("k", 0, 5000)])
    _rocpd(str(d / "b_results.db"), kernels=[("k", 100, 3100)])
    assert bench.trace_durations(str(d))["k"] == [5000, 3000, 1000]
    bench.print_trace_summary(str(d), last=2)
    head, row = capsys.readouterr().out.splitlines()
    assert "last 2" in head
    assert row.split()[:5] == ["3", "3.000", "1.000", "5.000", "2.000"]


def test_settle_runs_whole_synchronized_chunks_until_the_time_is_up(monkeypatch):
    import time

    import torch

    syncs = []
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: syncs.append(1))
    seen = []
    assert bench.settle(seen.append, 0.0) == 0 and not seen and not syncs
    t0 = time.perf_counter()
    n = bench.settle(lambda i: (seen.append(i), time.sleep(0.0005)), 20.0, chunk=8)
    assert (time.perf_counter() - t0) * 1e3 >= 20.0
    assert n > 0 and n % 8 == 0 and seen == list(range(n)) and len(syncs) == n // 8


def test_traffic_lookup_is_gated_on_the_source_hash(tmp_path, monkeypatch):
    rec = {"workload": "w", "M": 4, "flags": 0, "ws": True, "src_hash": bench.kernel_source_hash(),
           "traffic_bytes": 1234}
    stale = dict(rec, src_hash="0" * 16, traffic_bytes=99)
    plain = dict(rec, ws=False, traffic_bytes=777)
    (tmp_path / "k_w.md").write_text("# summary\n\ntraffic_record: " + json.dumps(stale) + "\n"
                                     "traffic_record: " + json.dumps(rec) + "\n"
                                     "traffic_record: " + json.dumps(plain) + "\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.lookup_traffic("w", 4, 0) == 1234
    assert bench.lookup_traffic("w", 4, 0, ws=False) == 777
    assert bench.lookup_traffic("w", 8, 0) is None
    (tmp_path / "k_w.md").write_text("traffic_record: " + json.dumps(stale) + "\n")
    assert bench.lookup_traffic("w", 4, 0) is None


def test_cpu_baseline_times_the_oracle_on_a_sample():
    from block_quantized_weight_amd import synth

    prob = synth.workload("u4_m1_k512_n256")
    out = bench.cpu_baseline(prob, 1, 0.2)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "columns" in out["sample"]
    assert out["single_thread"]["cores"] == 1 and out["single_thread"]["value"] > 0
    assert out["cpu_model"]


def test_committed_profiles_name_their_commands():
    """Every profiler summary gives the commands that made it, run on committed files."""
    pdir = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(pdir) if f.endswith((".md", ".txt"))]
    assert files
    for f in files:
        txt = open(os.path.join(pdir, f)).read()
        if f.startswith("counters_"):
            # instruction / occupancy counter summaries: the --pmc runs and their reader
            assert "rocprofv3 --pmc SQ_" in txt and "bench.py --counter-summary" in txt, f
        else:
            # per-kernel summaries: the kernel trace and the two traffic counter runs
            assert "rocprofv3 --kernel-trace --stats" in txt and "rocprofv3 --pmc FETCH_SIZE" in txt, f
        assert "_work" not in txt, f
        assert len(txt) < 16 * 1024, f
