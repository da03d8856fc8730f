"""Host logic of bench.py (CPU only): the algorithmic byte counts behind the
roofline figure, the counter summaries (per kernel and per call) and their
guard, and the one-GPU limit."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _shaped(B, K, V, dtype=np.uint16, temperature=None):
    """Arrays of the right shape; np.empty touches no pages."""
    T = np.full(B, 0.6, np.float32) if temperature is None else temperature
    return {"target": np.empty((B, K + 1, V), dtype), "temperature": T}


def test_config1_bytes_are_every_logit_once():
    # 64 rows x (6 target + 5 draft) positions x 151,936 bf16 logits
    by = bench.algorithmic_bytes(_shaped(64, 5, 151936))
    assert by["stats_kernel"] == 64 * 11 * 151936 * 2 == 213925888
    assert by["m_min"] > by["stats_kernel"]


def test_greedy_rows_skip_their_drafts():
    # config 3: 512 rows, half greedy (their drafts are never read)
    T = np.where(np.arange(512) < 256, 0.0, 0.8).astype(np.float32)
    by = bench.algorithmic_bytes(_shaped(512, 4, 128256, temperature=T))
    assert by["stats_kernel"] == 512 * 5 * 128256 * 2 + 256 * 4 * 128256 * 2 == 919339008


def test_fp32_logits_count_four_bytes():
    by = bench.algorithmic_bytes(_shaped(4, 4, 1024, dtype=np.float32))
    assert by["stats_kernel"] == 4 * 9 * 1024 * 4


def test_tree_bytes_count_the_drafts_of_nodes_with_children():
    par = np.asarray(W.TREE_60_DEPTH8, dtype=np.int32)
    N = par.size
    internal = np.unique(par[1:]).size
    d = {"target": np.empty((32, N, 151936), np.uint16), "temperature": np.full(32, 1.0, np.float32),
         "parents": np.broadcast_to(par, (32, N))}
    by = bench.tree_algorithmic_bytes(d)
    assert by["internal_nodes"] == 32 * internal
    assert by["stats_kernel"] == 32 * (N + internal) * 151936 * 2
    # greedy rows read no draft
    d["temperature"] = np.zeros(32, np.float32)
    assert bench.tree_algorithmic_bytes(d)["stats_kernel"] == 32 * N * 151936 * 2


def test_counter_summary_is_used_only_for_its_own_kernel_source(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "stats_kernel_B1K1V1_pmc.txt").write_text(
        "kernel_source_hash: 0123456789abcdef\nhbm_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    assert bench.traffic_from_profiles("B1K1V1") == 12345.0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "fedcba9876543210")
    assert bench.traffic_from_profiles("B1K1V1") is None
    assert bench.traffic_from_profiles("B2K2V2") is None


def test_whole_call_counters_sum_every_kernel_of_the_call(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "stats_kernel_B1K1V1_pmc.txt").write_text(
        "kernel_source_hash: 0123456789abcdef\n"
        "stats_kernel: 36 dispatches; read 1000 B, written 10 B; VALUBusy 50.0%\n"
        "hbm_bytes_per_launch: 1010\n"
        "merge_kernel: 36 dispatches; read 200 B, written 20 B; VALUBusy 40.0%\n"
        "finish_kernel: 36 dispatches; read 30 B, written 3 B; VALUBusy 4.0%\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    t = bench.call_traffic_from_profiles("B1K1V1")
    assert t == {"read": 1230.0, "written": 33.0, "kernels": ["finish_kernel", "merge_kernel", "stats_kernel"]}
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "fedcba9876543210")
    assert bench.call_traffic_from_profiles("B1K1V1") is None


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_median_of_three_and_host_facts():
    d = W.make(0)
    cb, ref = bench.cpu_baseline(d, 0.3)
    assert cb["kind"] == "oracle" and cb["unit"] == "positions/s" and len(cb["runs"]) == 3
    assert cb["value"] == sorted(cb["runs"])[1] or abs(cb["value"] - sorted(cb["runs"])[1]) < 0.1
    assert 1 <= cb["cores"] <= bench.CPU_THREADS
    assert cb["host"]["logical_cpus"] == os.cpu_count()
    assert len(ref) == d["target"].shape[0]


def test_oracle_comparison_counts_equal_and_differing_rows():
    d = W.make(0)
    _, ref = bench.cpu_baseline(d, 0.05)
    out = np.stack([r.tokens for r in ref]).astype(np.int32)
    nacc = np.array([r.n for r in ref], dtype=np.int32)
    c = bench.oracle_comparison(out, nacc, ref, d["uniforms"])
    assert c["rows"] == 4 and c["rows_equal"] == 4 and c["firm_rows_differing"] == 0
    b = next(k for k, r in enumerate(ref) if r.gap > 1e-3)
    out[b, ref[b].n] = (out[b, ref[b].n] + 1) % d["target"].shape[2]
    c = bench.oracle_comparison(out, nacc, ref, d["uniforms"])
    assert c["rows_equal"] == 3 and c["firm_rows_differing"] == 1
