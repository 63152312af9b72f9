"""Host logic of bench.py (no GPU): the one-GPU refusal, the source check that keeps stale
HBM-traffic records out of the report, and the rocprofv3 statistics summary."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    rec = {"traffic_bytes_per_launch": 1.5e9, "source_sha256": bench.sources_sha(bench.SPARSE_SOURCES)}
    path = tmp_path / "traffic_{workload}.json"
    (tmp_path / "traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.read_traffic("w") == 1.5e9
    rec["source_sha256"] = "0" * 64                     # taken on other kernel sources
    (tmp_path / "traffic_w.json").write_text(json.dumps(rec))
    assert bench.read_traffic("w") is None
    assert bench.read_traffic("missing") is None


def test_trace_summary(tmp_path, capsys):
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    (d / "p_kernel_stats.csv").write_text(
        "Name,Calls,TotalDurationNs,AverageNs,Percentage\n"
        '"void sla::sparse_attn_kernel<unsigned short, 128, 2, false, false>(sla::SparseArgs)",'
        "13,6520000,501538.5,58.6\n"
        '"void sla::(anonymous namespace)::helper(int)",2,9000,4500,0.1\n')
    out = tmp_path / "k.txt"
    bench.summarize_trace(str(tmp_path / "trace"), str(out), "rocprofv3 ... -- python bench.py")
    lines = out.read_text().splitlines()
    assert lines[1] == "# command: rocprofv3 ... -- python bench.py"
    row = lines[4].split()
    assert row[0] == "sla::sparse_attn_kernel<unsigned" and row[-3:] == ["13", "501.54", "58.60"]
    assert lines[5].split()[0] == "sla::helper" and lines[5].split()[-2] == "4.50"
