"""Host-side logic of bench.py that needs no GPU: the refusal of multi-GPU runs and the rules
that decide when committed HBM traffic counters may be reported beside a live measurement."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.fixture
def fake_tree(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// kernel source\n")
    rec = {"config_id": 3, "p": 0.9,
           "calls": {"quest_page_scores": {"bytes_per_launch": 34180000,
                                           "sources": {"k.hip": bench.source_digest(str(src))}}}}
    traffic = tmp_path / "traffic.json"
    traffic.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    return src, traffic


def test_traffic_is_reported_for_the_workload_it_was_taken_on(fake_tree):
    assert bench.measured_traffic("quest_page_scores", 3, 0.9) == 34180000


@pytest.mark.parametrize("call,config_id,p", [
    ("quest_page_scores", 2, 0.9),       # another workload
    ("quest_page_scores", 3, 0.8),       # another threshold
    ("twilight_sparse_decode", 3, 0.9),  # a call the counters did not cover
])
def test_traffic_is_withheld_elsewhere(fake_tree, call, config_id, p):
    assert bench.measured_traffic(call, config_id, p) is None


def test_traffic_is_withheld_once_a_kernel_source_changes(fake_tree):
    src, _ = fake_tree
    src.write_text("// kernel source, edited\n")
    assert bench.measured_traffic("quest_page_scores", 3, 0.9) is None
    src.unlink()
    assert bench.measured_traffic("quest_page_scores", 3, 0.9) is None


def test_missing_or_unreadable_counter_file_gives_none(fake_tree):
    _, traffic = fake_tree
    traffic.write_text("{not json")
    assert bench.measured_traffic("quest_page_scores", 3, 0.9) is None
    traffic.unlink()
    assert bench.measured_traffic("quest_page_scores", 3, 0.9) is None


def test_cpu_baseline_reports_the_threads_that_ran():
    """The host oracle baseline on the one-unit workload: both variants run, and the
    multi-threaded one counts only the threads that had a unit to work on."""
    from adaptive_top_sparse_amd import workloads
    w = workloads.make_workload(1)
    r = bench.cpu_baseline(w, 0.9, seconds=0.05)
    assert r["kind"] == "oracle" and r["unit"] == "candidate tokens/s"
    assert r["units_per_step"] == 1
    assert r["cores"] == 1
    assert r["value"] > 0 and r["single_thread"]["value"] > 0 and r["single_thread"]["cores"] == 1
    assert r["usable_cores"] >= 1 and r["cpu_model"]
