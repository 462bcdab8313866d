"""bench.py's host logic, without a GPU: the one-GPU guard, the traffic record's source
hash check (and that the committed records match the kernel source), the CPU description
of the baseline, the summary of timeline records and the choice of how a kernel is timed."""

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


def _rec(start, loop0, loop1, end, xcd, cu, tiles):
    # stamps in the 100 MHz clock's ticks (0.01 µs); HW_ID holds the CU index in bits 8-11
    return [start, loop0, loop1, end, cu << 8, xcd, tiles, 0]


def test_timeline_summary_of_synthetic_records():
    rec = [
        _rec(0, 100, 900, 1000, xcd=0, cu=1, tiles=4),      # unit A: 0-10 µs
        _rec(0, 100, 1800, 2000, xcd=1, cu=1, tiles=4),     # unit B: 0-20 µs
        _rec(1200, 1300, 2100, 2200, xcd=0, cu=1, tiles=4),  # unit A again after a 2 µs gap
    ]
    s = bench.timeline_summary(rec)
    assert s["workgroups"] == 3 and s["compute_units"] == 2
    assert abs(s["span_us"] - 22.0) < 1e-9
    assert abs(s["prologue_us_mean"] - 1.0) < 1e-9
    assert abs(s["loop_us_per_key_tile"] - (8 + 17 + 8) / 12) < 1e-9
    assert abs(s["epilogue_us_mean"] - 4 / 3) < 1e-9
    assert abs(s["gap_us_mean"] - 2.0) < 1e-9
    assert abs(s["transition_share"] - (3 + 4 + 2) / (40 + 2)) < 1e-9
    assert s["xcd_end_us"] == [22.0, 20.0] and s["unit_end_us_min"] == 20.0
    assert abs(s["tail_idle_share"] - (1 - 21 / 22)) < 1e-9
    # a workgroup that saw no key records its entry only: it counts as a zero-length visit
    s2 = bench.timeline_summary(rec + [[2100, 0, 0, 0, 1 << 8, 1, 0, 0]])
    assert s2["workgroups"] == 4 and abs(s2["gap_us_mean"] - 1.5) < 1e-9
    assert s2["xcd_end_us"] == [22.0, 21.0]
    assert abs(s2["prologue_us_mean"] - 1.0) < 1e-9


def test_traffic_records_were_taken_on_the_current_kernel_source():
    # the bench line's roofline.traffic comes from these records; a kernel change needs them retaken
    for dtype in ("fp8", "fp8_lean", "bf16"):
        rec = json.load(open(os.path.join(ROOT, "profiles", f"attn_fwd_{dtype}_gqa32k_hbm.json")))
        assert rec["kernel_source_hash"] == bench.kernel_hash(), dtype


class _FakeClock:
    """A stand-in for torch.cuda's events and spin kernel: each call of fn advances a GPU
    timeline by its kernel time; the host issue time is simulated by the test."""

    def __init__(self, kernel_ms):
        self.kernel_ms, self.gpu_ms, self.sleeps = kernel_ms, 0.0, []
        outer = self

        class Event:
            def __init__(self, enable_timing=False):
                self.t = None

            def record(self, stream=None):
                self.t = outer.gpu_ms

            def elapsed_time(self, other):
                return other.t - self.t

        class Cuda:
            pass

        self.cuda = Cuda()
        self.cuda.Event = Event
        self.cuda.synchronize = lambda: None
        self.cuda._sleep = lambda cycles: self.sleeps.append(cycles)

    host_s = 0.0

    def fn(self):  # each call takes the host 50 us to issue
        self.gpu_ms += self.kernel_ms
        _FakeClock.host_s += 50e-6


def test_short_kernels_are_queued_behind_a_spin_and_long_ones_are_not(monkeypatch):
    monkeypatch.setattr(bench, "spin_cycles_per_ms", lambda torch: 2.0e6)
    monkeypatch.setattr(bench.time, "perf_counter", lambda: _FakeClock.host_s)
    for kernel_ms, spins in ((0.1, True), (1.2, False)):
        fake = _FakeClock(kernel_ms)
        mean, median = bench.time_kernel(fake.fn, 20, 3, None, fake)
        assert abs(mean - kernel_ms) < 1e-9 and abs(median - kernel_ms) < 1e-9
        assert bool(fake.sleeps) == spins
        if spins:  # long enough for the issue of every timed call, and bounded
            assert 2.0e6 * (20 * 0.05) <= fake.sleeps[0] <= 2.0e6 * 300
