"""Host logic of bench.py (CPU only): kernel-name normalisation, the HBM-byte
summary built from two profiler databases and a calibration copy, the source
hash gate on reported traffic, and the single-GPU guard."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_short_kernel_name():
    assert bench.short_kernel_name("void qg::gemm_x<1, 2>(unsigned char const*, int)") == "gemm_x<1, 2>"
    assert bench.short_kernel_name("qg::skinny_kernel<1, 1, 1, 0, 2>(args)") == "skinny_kernel<1, 1, 1, 0, 2>"
    assert bench.short_kernel_name("plain") == "plain"


def _db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table pmc_events (name text, dispatch_id int, counter_name text, "
                "counter_value real)")
    con.executemany("insert into pmc_events values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_pmc_summary_scales_by_the_copy_kernel(tmp_path):
    mib = 8
    copy = "at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)"
    kern = "void qg::gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1>(args)"
    # the copy reads and writes 8 MiB; its FETCH_SIZE reads back half (KiB), WRITE_SIZE all
    fetch = [(copy, 1, "FETCH_SIZE", mib * 1024 / 2), (copy, 2, "FETCH_SIZE", mib * 1024 / 2),
             # one dispatch reported as two per-XCD instances that must be summed
             (kern, 3, "FETCH_SIZE", 100.0), (kern, 3, "FETCH_SIZE", 50.0),
             (kern, 4, "FETCH_SIZE", 250.0)]
    write = [(copy, 1, "WRITE_SIZE", mib * 1024.0), (copy, 2, "WRITE_SIZE", mib * 1024.0),
             (kern, 3, "WRITE_SIZE", 64.0), (kern, 4, "WRITE_SIZE", 64.0)]
    fdb, wdb, out = tmp_path / "f.db", tmp_path / "w.db", tmp_path / "t.json"
    _db(fdb, fetch)
    _db(wdb, write)
    bench.pmc_summary(str(fdb), str(wdb), str(out), mib)
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    k = t["kernels"]["gemm_q4k_lds_kernel<1, 1, 2, 4, false, 2, 4, 1>"]
    assert k["dispatches"] == 2
    assert k["fetch_kib"] == pytest.approx(200.0)           # (150 + 250) / 2
    assert k["read_bytes"] == round(200.0 * 1024 * 2.0)
    assert k["write_bytes"] == round(64.0 * 1024 * 1.0)
    assert t["source_sha256"] == bench.source_hash()


def test_pmc_summary_needs_the_copy_kernel(tmp_path):
    fdb, wdb = tmp_path / "f.db", tmp_path / "w.db"
    _db(fdb, [("k", 1, "FETCH_SIZE", 1.0)])
    _db(wdb, [("k", 1, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.pmc_summary(str(fdb), str(wdb), str(tmp_path / "t.json"), 8)


def test_traffic_only_while_sources_hash_the_same(tmp_path, monkeypatch):
    t = {"source_sha256": bench.source_hash(),
         "kernels": {"k<1>": {"read_bytes": 100, "write_bytes": 20}}}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(t))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(p))
    assert bench.traffic_for("k<1>") == 120
    assert bench.traffic_for("other<2>") is None
    t["source_sha256"] = "0" * 64
    p.write_text(json.dumps(t))
    assert bench.traffic_for("k<1>") is None
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "missing.json"))
    assert bench.traffic_for("k<1>") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
