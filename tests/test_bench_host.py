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


def _receipt(**over):
    out = {"metric": bench.METRIC, "value": 612.3, "unit": "TOPS", "n_gpus": 1, "steps": 100,
           "warmup": 10, "ms_per_step": 0.168, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "int8", "data": "synthetic (seeded)",
           "config": {"workload": "long-prompt gate+up projection at one 512-row chunk: quantise bf16 "
                                  "x [512x4096] + Q4_K GEMM 4096->24576",
                      "M": 512, "K": 4096, "N": 24576, "fmt": "Q4_K", "projections": [[4096, 24576]]},
           "prefill_tok_s": 3.0e6, "quant_us": 5.1, "gemm_us": 160.2,
           "step_ms_p10_p50_p90": [0.16, 0.17, 0.18], "wall_s_timed": 0.02,
           "roofline": {"bound": "mfma", "kernel": "gemm_q4k_mix_kernel",
                        "achieved": 643.1, "peak": 5000.0, "unit": "TOPS", "frac": 0.1286,
                        "traffic": 123456789, "avg_launch_us": 160.2, "ops_per_launch": 103079215104},
           "cpu_baseline": {"value": 0.0958, "unit": "TOPS", "cores": 16, "nproc": 16,
                            "cpu_model": "AMD EPYC 9575F 64-Core Processor", "kind": "oracle",
                            "sample": "the whole step (512x4096->24576 Q4_K, activation quantisation "
                                      "included) x10 in 12.3 s", "tok_s": 470.0},
           "lm_head": {"kernel_us": 89.1, "gbps": 5734.2, "frac_hbm": 0.7168},
           "large_m": {f"c4_{s}_M{m}": 0.1234 for m in (512, 2048, 8192) for s in ("gate_up", "down")} |
                      {f"c3_{s}_M{m}": 0.1234 for m in (512, 4096) for s in ("gate_up", "down", "attn_out")},
           "layer_tok_s": {f"config{c}_M{m}": 1234567.8 for c, ms in ((2, (512,)), (3, (512, 4096)),
                                                                    (4, (512, 2048, 8192))) for m in ms},
           "provenance": {"git_sha": "0123456789ab", "source_sha256": "0123456789abcdef",
                          "rocm": "7.2.0", "hip": "7.0.51831", "torch": "2.10.0+rocm7.0",
                          "gpu": "AMD Instinct MI355X gfx950:sramecc+:xnack-", "sclk_mhz_measured": 2100.0,
                          "cu": 256}}
    out.update(over)
    return out


def test_compact_line_is_the_receipt_and_fits():
    line = bench.compact_line(_receipt())
    assert len(line.encode()) <= bench.LINE_LIMIT
    d = json.loads(line)
    for k in bench.REQUIRED:
        assert k in d, k
    assert d["config"]["projections"] == [[4096, 24576]]
    assert d["roofline"]["unit"] == "TOPS" and d["roofline"]["frac"] == pytest.approx(643.1 / 5000, abs=1e-4)
    assert d["cpu_baseline"]["cpu_model"] and d["cpu_baseline"]["cores"] == 16
    assert "tables" not in d and "step_ms_p10_p50_p90" not in d


def test_compact_line_fails_closed():
    r = _receipt()
    del r["roofline"]
    with pytest.raises(KeyError):
        bench.compact_line(r)
    r = _receipt()
    del r["roofline"]["traffic"]
    with pytest.raises(KeyError):
        bench.compact_line(r)
    r = _receipt()
    del r["cpu_baseline"]["cpu_model"]
    with pytest.raises(KeyError):
        bench.compact_line(r)
    with pytest.raises(ValueError):
        bench.compact_line(_receipt(data="x" * 3000))


def test_compact_line_drops_summaries_before_the_limit():
    """Over the limit, the optional summaries go (the last first); the receipt stays."""
    r = _receipt()
    r["layer_tok_s"] = {f"set{i}": 1234567.8 for i in range(40)}
    line = bench.compact_line(r)
    d = json.loads(line)
    assert len(line.encode()) <= bench.LINE_LIMIT
    assert "layer_tok_s" not in d and "provenance" in d
    for k in bench.REQUIRED:
        assert k in d, k


def test_provenance_helpers():
    assert bench.cpu_model()
    assert bench.usable_cpus() >= 1
    assert len(bench.source_hash()) == 64
