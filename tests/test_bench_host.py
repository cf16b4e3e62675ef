"""Host-side logic of bench.py that needs no GPU: the refusal of multi-GPU runs, the rules
that decide when committed HBM traffic counters may be reported beside a live measurement,
the algorithmic byte model behind every roofline fraction, and the CPU baseline's fields."""
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


def _fake_step(B, Hq, Hkv, seq, stride, budget, sel=None, kept=None):
    """CPU stand-ins for the device cache and step buffers that bench.stage_bytes reads."""
    import types
    import torch
    c = types.SimpleNamespace(B=B, Hq=Hq, Hkv=Hkv, seq_lens=torch.tensor(seq, dtype=torch.int32),
                              cand_stride_pages=stride, budget=budget)
    buf = types.SimpleNamespace(kept_count=torch.tensor(kept, dtype=torch.int32))
    if budget is not None:
        pages = torch.zeros((B, Hkv, budget), dtype=torch.int32)
        count = torch.zeros((B, Hkv), dtype=torch.int32)
        for (b, g), pg in sel.items():
            pages[b, g, :len(pg)] = torch.tensor(pg, dtype=torch.int32)
            count[b, g] = len(pg)
        buf.sel_pages, buf.sel_count = pages, count
    return c, buf


def test_algorithmic_bytes_follow_the_per_unit_model_with_a_quest_base():
    # B = 1, 8 query heads over 2 KV heads, d = 128, a 100-token sequence (7 pages, the last
    # holding 4 tokens), 3 pages selected per KV head, 20 + 30 tokens kept. Per-unit bytes:
    # 512 per page-head of bounds and 8 per page-head of fp64 score written / read, 80 per
    # candidate token-head of codes and {scale, zero}, 8 per candidate slot and query head of
    # fp32 weight written and read, 4 per kept id written (top-p) and 4 read (decode), 512
    # per kept token-head of K and V, and 256 per query head for q (o in the decode too).
    c, buf = _fake_step(1, 8, 2, [100], 3, 3, sel={(0, 0): [0, 3, 6], (0, 1): [1, 2, 5]},
                        kept=[[20, 30]])
    out, cand, kept = bench.stage_bytes(c, buf, 128)
    assert cand == (16 + 16 + 4) + (16 + 16 + 16) and kept == 50
    q = 8 * 256
    assert out["quest_page_scores"] == 7 * 2 * 512 + q + 7 * 2 * 8
    assert out["quest_top_pages"] == 7 * 2 * 8 + 6 * 4
    assert out["twilight_estimate_topp"] == 84 * 80 + 84 * 4 * 8 + q + 50 * 4
    assert out["twilight_sparse_decode"] == 50 * (512 + 4) + 2 * q


def test_algorithmic_bytes_without_a_selector_count_every_token():
    # B = 2 sequences of 1000 and 37 tokens, MHA with 2 heads, d = 64: every token is a
    # candidate (64/2 bytes of codes + 2 groups x 4 bytes of {scale, zero} = 40 bytes per
    # token-head), no Quest calls
    c, buf = _fake_step(2, 2, 2, [1000, 37], 63, None, kept=[[500, 400], [37, 10]])
    out, cand, kept = bench.stage_bytes(c, buf, 64)
    assert set(out) == {"twilight_estimate_topp", "twilight_sparse_decode"}
    assert cand == 2 * 1000 + 2 * 37 and kept == 947
    q = 2 * 2 * 128
    assert out["twilight_estimate_topp"] == cand * 40 + cand * 1 * 8 + q + kept * 4
    assert out["twilight_sparse_decode"] == kept * (256 + 4) + 2 * q
