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


def test_sample_units_cover_the_batch():
    for n in (8, 16):
        units = bench.sample_units(8, 8, n)
        assert len(set(units)) == n
        assert sorted(set(b for b, _ in units)) == list(range(8))
        assert all(0 <= kv < 8 for _, kv in units)


def test_host_threads_reports_the_affinity_mask():
    cores, blas = bench.host_threads()
    assert cores == len(os.sched_getaffinity(0)) and blas >= 1


class _FakeStep:
    """A tiny long-context-shaped step for the CPU baseline harness."""

    def __init__(self, b, hq, hkv, d, L, s, budget):
        self.config = {"batch": b, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
                       "seq_len": L, "page_size": s, "budget_tokens": budget}
        units = b * hkv
        self.kv_bytes = units * (L // s) * 2 * d * 2 + units * (budget // s) * s * 2 * d * 2


def _fake_data(step, planted_err=0.0):
    """Inputs plus 'device' results computed by the oracle itself (CPU
    tensors), optionally with an error planted in the dense output."""
    import numpy as np
    import torch
    import oracle
    from oracle import quest as oquest
    from decode_attention_folded_amd import workloads
    cfg = step.config
    b, hq, hkv, d, L, s = (cfg[k] for k in ("batch", "num_q_heads", "num_kv_heads", "head_dim",
                                            "seq_len", "page_size"))
    case = workloads.dense_case(77, b, hq, hkv, d, L, [L] * b, plant_pages=2, with_new=True)
    k2, v2 = oracle.append_kv(case.k, case.v, case.seqlens, case.k_new, case.v_new)
    dense = oracle.decode_attention(case.q, k2, v2, case.seqlens, 1 / np.sqrt(d))
    meta = oquest.build_metadata(k2, case.seqlens, s, L // s)
    idx = oquest.select_pages(oquest.page_scores(case.q, meta, case.seqlens, s), case.seqlens,
                              s, cfg["budget_tokens"] // s)
    quest = oquest.sparse_decode_attention(case.q, k2, v2, case.seqlens, idx, s, 1 / np.sqrt(d))
    dense[0, 0, 0] += planted_err
    t = torch.from_numpy
    return {"q": t(case.q), "k": t(k2), "v": t(v2), "k_new": t(case.k_new),
            "v_new": t(case.v_new), "dense_out": t(dense.astype(np.float16)),
            "quest_out": t(quest.astype(np.float16)), "idx": t(idx)}


def test_long_context_cpu_baseline_reports_parity():
    step = _FakeStep(2, 8, 2, 64, 512, 16, 128)
    c = _fake_data(step)
    units = bench.sample_units(2, 2, 3)
    r = bench.long_context_cpu_baseline(step, c, units)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    assert r["host_cores"] == len(os.sched_getaffinity(0)) and r["blas_threads"] == 1
    p = r["parity"]
    # the fp16-rounded oracle results agree with the fp64 oracle within rounding
    assert p["dense_max_abs_err"] <= 1e-3 and p["quest_max_abs_err"] <= 1e-3
    assert p["idx_exact"] == p["idx_units"] == 3
    assert p["idx_near_tie_swaps"] == 0 and p["idx_rule_violations"] == 0


def test_long_context_cpu_baseline_sees_a_wrong_output():
    step = _FakeStep(1, 4, 1, 64, 256, 16, 64)
    c = _fake_data(step, planted_err=0.5)
    r = bench.long_context_cpu_baseline(step, c, [(0, 0)])
    assert r["parity"]["dense_max_abs_err"] >= 0.4
