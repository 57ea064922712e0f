"""CPU checks of bench.py's host logic (no GPU): the one-GPU refusal, the
hash-gated counter traffic, the step-token recipe and the CPU-oracle
baseline's report."""

import json
import os
import subprocess
import sys

import numpy as np

import bench
from bit_kv_cache_decode_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr + r.stdout


def test_traffic_is_used_only_for_the_kernel_source_it_was_measured_on(monkeypatch, tmp_path):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel_source_sha256": bench.kernel_hash(),
                             "workload": "llama2_7b_layer", "bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("llama2_7b_layer") == 123
    assert bench.measured_traffic("llama2_13b_layer") is None        # another workload
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 64)     # source changed
    assert bench.measured_traffic("llama2_7b_layer") is None
    f.write_text("not json")
    assert bench.measured_traffic("llama2_7b_layer") is None


def test_step_tokens_end_on_the_workload_or_append_one_more():
    w = wl.generate(2, batch=2)
    r0, k_new, v_new = bench.step_tokens(w)
    assert np.array_equal(r0, w.r_len - 1)
    last = w.lengths - 1
    for b in range(2):                       # the appended token is the last one
        assert np.array_equal(k_new[b], w.k[b, :, last[b]])
        assert np.array_equal(v_new[b], w.v[b, :, last[b]])
    w4 = wl.generate(4, batch=8)             # ragged: some windows are empty
    assert np.any(w4.r_len == 0)
    r4, k4, v4 = bench.step_tokens(w4)
    assert np.array_equal(r4, w4.r_len) and np.all(r4 + 1 <= w4.config.residual)
    assert k4.shape == (8, w4.config.heads, w4.config.head_dim) and k4.dtype == np.float16


def test_cpu_baseline_reports_the_oracle_and_its_threads():
    w = wl.generate(1)
    r = bench.cpu_baseline(w, 0.3)
    assert r["kind"] == "oracle" and r["unit"] == "query-heads/s"
    assert r["value"] > 0 and "steps" in r["sample"]
    assert r["cores"] >= 1 and r["host_cpus"] == os.cpu_count()
    assert r["affinity_cpus"] == len(os.sched_getaffinity(0))
    assert r["cores"] == (r["blas_threads"] or 1)


def test_oracle_sample_times_decode_and_flush():
    w = wl.generate(3, batch=2)
    r = bench.oracle_sample(w, 4, 1, flush=True)
    assert r["heads"] == 4 and r["decode_s"] > 0 and r["query_heads_per_s"] > 0
    assert r["flush_s"] > 0 and r["flushes_per_s"] > 0


def test_every_other_workload_is_listed_once():
    """The decode of every workload besides the headline one, long context
    at both widths."""
    assert sorted(bench.EXTRA_WORKLOADS, key=str) == sorted(
        [(1, None), (3, None), (4, None), (5, 2), (5, 4)], key=str)
    assert set(bench.ORACLE_SAMPLE_HEADS) == {1, 2, 3, 4, 5}
