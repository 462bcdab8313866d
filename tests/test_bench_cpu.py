"""bench.py's host logic, without a GPU: the one-GPU guard, the traffic record's source
hash check and the CPU description of the baseline."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_reported_only_for_the_profiled_kernel_source(monkeypatch):
    path = os.path.join(ROOT, "profiles", "attn_fwd_fp8_gqa32k_hbm.json")
    rec = json.load(open(path))
    monkeypatch.setattr(bench, "kernel_hash", lambda: rec["kernel_source_hash"])
    assert bench.hbm_traffic("gqa32k", "fp8") == rec["hbm_bytes_per_launch"]
    assert rec["hbm_bytes_per_launch"] > rec["algorithmic_bytes_per_launch"] > 0
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.hbm_traffic("gqa32k", "fp8") is None
    assert bench.hbm_traffic("no-such-workload", "fp8") is None


def test_kernel_hash_covers_the_attention_sources():
    h = bench.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert "fp8_causal_prefill_amd/csrc/attn_fwd.hip" in bench.KERNEL_SOURCES


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
