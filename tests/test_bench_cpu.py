"""Host-side checks of bench.py: the one-GPU guard and the lookup of the
counter-measured HBM traffic of a stage (no GPU needed)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


def _write_summary(root, digest, workloads):
    os.makedirs(os.path.join(root, "profiles"))
    blob = json.dumps({"kernel_source_digest": digest, "workloads": workloads})
    with open(os.path.join(root, "profiles", "hbm_traffic_counters.md"), "w") as f:
        f.write("# counters\n\n```json\n" + blob + "\n```\n")


def test_counter_traffic_is_taken_per_stage(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "d1")
    _write_summary(str(tmp_path), "d1", {
        "quest128k": {"stages": {"append_score": {"bytes_per_call": 111},
                                 "select_sparse_attention": {"bytes_per_call": 222}}},
        "paged": {"stages": {"attention": {"bytes_per_call": 333}}},
    })
    assert bench.counter_traffic("quest128k", "append_score") == 111
    assert bench.counter_traffic("quest128k", "select_sparse_attention") == 222
    assert bench.counter_traffic("paged", "attention") == 333
    # a stage or workload the counters did not cover
    assert bench.counter_traffic("quest128k", "attention") is None
    assert bench.counter_traffic("exaone30", "attention") is None


def test_counter_traffic_needs_the_same_kernel_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "now")
    _write_summary(str(tmp_path), "then", {"paged": {"stages": {"attention": {"bytes_per_call": 1}}}})
    assert bench.counter_traffic("paged", "attention") is None


def test_counter_traffic_without_a_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("paged", "attention") is None


@pytest.mark.parametrize("name", ["attention_impl.h", "topk.h", "quest_kernels.hip"])
def test_digest_follows_the_code_not_the_comments(tmp_path, name):
    import shutil
    src = os.path.join(ROOT, "decode_attention_folded_amd", "csrc")
    dst = tmp_path / "decode_attention_folded_amd" / "csrc"
    shutil.copytree(src, dst)
    before = bench.kernel_source_digest(str(tmp_path))
    assert before == bench.kernel_source_digest(ROOT)
    with open(dst / name, "a") as f:
        f.write("\n// a comment\n/* and a\n   block comment */\n")
    assert bench.kernel_source_digest(str(tmp_path)) == before
    with open(dst / name, "a") as f:
        f.write("\nstatic const int digest_probe = 1;\n")
    assert bench.kernel_source_digest(str(tmp_path)) != before
