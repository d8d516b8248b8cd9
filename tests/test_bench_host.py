"""Host-side pieces of bench.py (no GPU): the metric names the workload it measures, and the HBM
traffic of a kernel class is taken from the counter summaries under profiles/ only for the workload
and the sources the counters were taken on."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_metric_names_the_measured_workload():
    assert bench.metric_name(bench.WORKLOADS["gpt2-124m"]) == \
        "training tokens/sec + bf16 MFU, GPT-2 124M B=16 T=1024 on 1 MI355X"
    assert "GPT-2 1558M" in bench.metric_name(bench.WORKLOADS["gpt2-1558m"])


def test_parameter_counts_match_the_printed_one():
    # the 1558M count printed in the training log of "Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672"
    assert bench.num_params(bench.WORKLOADS["gpt2-1558m"]) == 1_557_686_400
    assert bench.num_params(bench.WORKLOADS["gpt2-124m"]) == 124_475_904


def test_traffic_only_for_the_matching_workload_and_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    digest = bench.sources_sha256()
    (prof / "t.md").write_text(
        f"TRAFFIC workload=gpt2-124m class=gemm_fc fetch_bytes=100 write_bytes=20 sources_sha256={digest}\n"
        f"TRAFFIC workload=gpt2-124m class=adamw fetch_bytes=1 write_bytes=2 sources_sha256=stale\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "sources_sha256", lambda: digest)
    assert bench.measured_traffic("gemm_fc", "gpt2-124m") == 120
    assert bench.measured_traffic("gemm_fc", "gpt2-350m") is None   # other workload
    assert bench.measured_traffic("adamw", "gpt2-124m") is None     # sources changed since
    assert bench.measured_traffic("gemm_qkv", "gpt2-124m") is None  # no counters for the class
