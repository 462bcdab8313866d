"""Benchmark: causal prefill attention TFLOP/s on one MI355X, FP8 (e4m3) and BF16.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa32k] [--no-cpu]

Workload (default ``gqa32k``): B=1, Hq=32, Hkv=8, S=32768, D=128, causal, Q/K/V
~ N(0, 1) float32 from seed, resident in HBM before timing. One FP8 step is the
whole hot path: quantize Q, K and V to e4m3 with per-128-token scales, then the
FP8 attention kernel. One BF16 step is the BF16 attention kernel on bfloat16
inputs. FLOPs follow the FlashAttention causal convention, 2 (Dqk + Dv) S^2 / 2 per
(batch, query head); softmax work is not counted.

Prints one JSON line. ``value`` is FP8 whole-step throughput; the attention kernel
alone is timed with HIP events on the stream it runs on and reported against the
datasheet dense FP8 peak in ``roofline``; the opt-in lean-probability FP8 mode is
reported in ``fp8_lean`` and BF16 in ``bf16``; ``range`` times the range entry points
(chunked prefill, split-KV with the merge kernel and its HBM roofline) and ``varlen`` a
packed batch of eight sequences of 256 to 16384 tokens on the same tensors. The CPU baseline times the fp64 oracle
on a bounded sample (whole query heads, about 15 s) on the host cores; the heads it
computed also give a full-size parity figure (``sampled_rel_l2_fp8``). ``cold_caches``
times the FP8 kernel again, each launch after a 512 MiB fill that evicts its inputs from
L2 and the Infinity Cache (median and mean of twice ``--steps`` launches).

``sustained`` runs each headline kernel back to back for a few seconds after the clock
has settled and reports, next to its time, the median shader clock, the socket power,
the energy per call and the fraction of the window the board spent at its power limit
(amdsmi telemetry; null with the reason when the driver does not provide it); its
``structured_inputs`` part does the same for the FP8 kernels at the 16K activation-like
shape on Gaussian, activation-like (with and without rotation) and rising-score inputs.
The activation-like workload's record in ``other_workloads`` carries, besides times, its
error figures with and without rotation (kernel against the oracle on the codes it read,
input quantization against unquantized inputs), computed in the CPU leg.

``--operand-zeros`` runs only the headline FP8 exact, FP8 lean and BF16 kernels with Q, K,
V or all three zeroed, each under the sustained telemetry, to show how the operands' bits
set the clock the board holds. ``--isa-costs`` runs only the instruction-cost probe built next to the library
(fp8_causal_prefill_amd/isa_cost: cycles per matrix instruction for e4m3 and e2m1
operands, SIMD cycles per vector instruction the softmax uses, and how matrix and
vector instructions of one wave overlap) and prints its figures as one JSON line.
``--isa-energy`` launches the same probe's kernels (fp8_causal_prefill_amd/libisa_cost.so)
on every compute unit, one instruction class at a time, each back to back under the
sustained telemetry, and prints the power, clock and energy per instruction of each class
over that of waves that only sleep. ``--timeline`` runs the headline-shape kernels (or
``--workload``'s) once each from the timeline build (fp8_causal_prefill_amd/libzyfa_timeline.so)
and prints where each launch's time goes: every workgroup's prologue, key-tile loop and
epilogue, the gaps between workgroups on a compute unit, and when each XCD goes idle.
"""

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X datasheet dense peaks (256 CUs x 2.4 GHz, an MFMA issued every cycle), TFLOP/s
PEAK_FP8 = 5033.2
PEAK_BF16 = 2516.6
PEAK_HBM_GBS = 8000.0

KERNEL_SOURCES = ["fp8_causal_prefill_amd/csrc/attn_fwd.hip", "fp8_causal_prefill_amd/csrc/device.h"]


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def hbm_traffic(workload_name, dtype):
    """Measured HBM bytes per attention launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{dtype}_{workload_name}_hbm.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def time_loop(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, q, k, v, target_s=15.0):
    """Time the fp64 oracle on a bounded sample of the workload: whole query heads
    (quantize + dequantize the head's Q and its KV head, then causal attention over
    all S rows), taken in order from head 0 until about target_s seconds are spent.
    Returns the baseline record and, per sampled head, the oracle output."""
    from oracle import causal_attention, dequantize_blocks, quantize_blocks
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        blas_threads = 1
    available = len(os.sched_getaffinity(0))
    cores = min(blas_threads, available)  # the threads the oracle's BLAS calls actually run on
    group = w.Hq // w.Hkv
    refs = {}
    flops = 0.0
    t0 = time.perf_counter()
    for hq in range(w.Hq):
        hkv = hq // group
        parts = [quantize_blocks(x[:1, h:h + 1], w.scale_block) for x, h in ((q, hq), (k, hkv), (v, hkv))]
        deq = [dequantize_blocks(c, s, w.scale_block) for c, s in parts]
        o, _ = causal_attention(deq[0], deq[1], deq[2], w.softmax_scale)
        refs[hq] = o[0, 0]
        flops += 2.0 * (w.Dqk + w.Dv) * w.S * (w.S + 1) / 2
        if time.perf_counter() - t0 >= target_s:
            break
    secs = time.perf_counter() - t0
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "host_cores_available": available, "blas_threads": int(blas_threads), "cpu_model": cpu_model(),
            "sample": f"fp64 oracle on {len(refs)} of {w.B * w.Hq} query heads of the same workload (batch 0, "
                      f"heads 0..{len(refs) - 1}, all {w.S} rows each: quantize, dequantize, causal attention); "
                      f"{secs:.1f} s",
            "seconds": round(secs, 3)}, refs


def time_kernel(fn, steps, warmup, stream, torch):
    """Mean and median milliseconds of fn() from HIP events on the stream it launches on.
    Issuing a call from Python (argument checks, two event records) takes the host tens of
    microseconds. Calls whose kernels run ten times longer or more queue up by themselves
    after two untimed launches. Shorter ones would leave the GPU waiting for the host, and
    events recorded as they are issued would time part of the host's work: those calls are
    queued behind a spin kernel that keeps the stream busy until all of them are issued, so
    that each event pair brackets its own launch, run back to back with the others. (Longer
    kernels are not queued that way: a burst of them after the idle spin runs a few percent
    slower than the same kernels back to back, as the board's power control catches up.)"""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    n0 = min(steps, 8)
    t0 = time.perf_counter()
    for e0, e1 in ev[:n0]:
        e0.record(stream)
        fn()
        e1.record(stream)
    host_ms = 1e3 * (time.perf_counter() - t0) / n0  # issue time per call (the queue is not full)
    torch.cuda.synchronize()
    kernel_ms = min(a.elapsed_time(b) for a, b in ev[:n0])
    rate = spin_cycles_per_ms(torch) if kernel_ms < 10.0 * host_ms else None
    if rate is not None:
        backlog_ms = min(2.0 + 3.0 * host_ms * steps, 300.0)  # margin for a clock faster than at calibration
        torch.cuda._sleep(int(backlog_ms * rate))
    else:
        fn()
        fn()
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    return float(np.mean(ms)), float(np.median(ms))


_SPIN_CYCLES_PER_MS = None


def spin_cycles_per_ms(torch):
    """Counter ticks per millisecond of torch's spin kernel on this GPU, measured once
    (None if the measurement is implausible)."""
    global _SPIN_CYCLES_PER_MS
    if _SPIN_CYCLES_PER_MS is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(2_000_000)
        e1.record()
        torch.cuda.synchronize()
        rate = 2_000_000 / max(e0.elapsed_time(e1), 1e-6)
        # a counter between 10 MHz and 10 GHz; anything else and the calls go unqueued
        _SPIN_CYCLES_PER_MS = rate if 1e4 <= rate <= 1e7 else False
    return _SPIN_CYCLES_PER_MS or None


class Telemetry:
    """Shader clock, socket power and energy of the GPU behind cuda:0, read from the
    driver's metrics table through amdsmi (ZYFA, "Throughput on Captured Activations at
    Sustained Clocks": the clock a kernel settles to under the board's power limit decides
    its throughput, so it is reported next to it). The table refreshes about once a
    second, so readings are taken over windows of a few seconds."""

    def __init__(self, torch):
        self.smi = None
        self.error = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            handle = handles[0] if len(handles) == 1 else None
            props = torch.cuda.get_device_properties(0)
            bus = getattr(props, "pci_bus_id", None)
            if bus is not None:
                for h in handles:  # match cuda:0 to its PCI address when the driver lists several GPUs
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                    if int(bdf.split(":")[1], 16) == int(bus) and int(bdf.split(":")[0], 16) == int(
                            getattr(props, "pci_domain_id", 0)):
                        handle = h
            if handle is None:
                raise RuntimeError(f"cannot tell which of {len(handles)} GPUs is cuda:0")
            self.smi, self.h = amdsmi, handle
            self.power_limit_w = amdsmi.amdsmi_get_power_info(handle).get("power_limit", 0) / 1e6
        except Exception as e:  # telemetry is optional: the bench line records why it is missing
            self.error = repr(e)

    def read(self):
        m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
        e = self.smi.amdsmi_get_energy_count(self.h)
        clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, int) and c > 0]
        return {"gfxclk": float(np.mean(clks)) if clks else None,
                "energy_j": e["energy_accumulator"] * e["counter_resolution"] * 1e-6,
                "ts_ns": e["timestamp"],  # the energy reading's own time stamp, nanoseconds
                "ppt": m.get("ppt_residency_acc"), "thm": m.get("socket_thm_residency_acc"),
                "acc": m.get("accumulation_counter")}


def sustained(tel, fn, flops, peak, settle_s, window_s, stream, torch):
    """Run fn back to back: settle_s seconds for the clock to reach its steady state under
    the power limit, then window_s seconds timed with HIP events on the kernel's stream
    while the telemetry is sampled. Power, clock and the power-limited fraction are taken
    between the first and the last refresh of the metrics table inside the window (readings
    between refreshes repeat the previous one). Returns the kernel time, throughput, median
    shader clock, mean socket power, energy per call and the fraction of the window that the
    board spent held at its power limit (or its thermal limit)."""
    import threading
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            samples.append(tel.read())
            stop.wait(0.02)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    ev = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < window_s:
        for _ in range(10):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
    stop.set()
    th.join()
    ms = float(np.mean([x.elapsed_time(y) for x, y in ev]))
    rec = {"calls": len(ev), "ms": ms, "tflops": flops / ms / 1e9, "frac": flops / ms / 1e9 / peak,
           "power_limit_w": tel.power_limit_w}
    # distinct table refreshes, skipping the first reading (taken before the window's launches)
    fresh = []
    for s in samples[1:]:
        if not fresh or s["ts_ns"] != fresh[-1]["ts_ns"]:
            fresh.append(s)
    if fresh and fresh[0]["ts_ns"] == samples[0]["ts_ns"]:
        fresh = fresh[1:]
    rec["refreshes"] = len(fresh)
    clks = [s["gfxclk"] for s in fresh if s["gfxclk"] is not None]
    rec["gfxclk_mhz_median"] = float(np.median(clks)) if clks else None
    if len(fresh) >= 2:
        a, b = fresh[0], fresh[-1]
        watts = (b["energy_j"] - a["energy_j"]) / ((b["ts_ns"] - a["ts_ns"]) * 1e-9)
        rec["socket_power_w"] = watts
        rec["energy_per_call_j"] = watts * ms * 1e-3
        if None not in (a["ppt"], b["ppt"], a["acc"], b["acc"]) and b["acc"] > a["acc"]:
            rec["power_limited_fraction"] = (b["ppt"] - a["ppt"]) / (b["acc"] - a["acc"])
            if a["thm"] is not None and b["thm"] is not None:
                rec["thermal_limited_fraction"] = (b["thm"] - a["thm"]) / (b["acc"] - a["acc"])
    return rec


def structured_sustained(tel, window_s, stream, torch, zy):
    """The sustained-clock measurement on inputs of different structure at one shape, the
    activation-like workload's (B=1, Hq=32, Hkv=8, S=16384, D=128): Gaussian inputs, the
    activation-like inputs without and with the 128-point rotation of Q and K, and rising
    scores (the lazy reference keeps moving). ZYFA, "Dependence of the Shader Clock on
    Operand Values" and "Throughput on Captured Activations at Sustained Clocks": the clock
    the board holds depends on the operands, so the same kernel is measured on each. FP8
    exact on every input set, lean on the Gaussian and rotated activation-like ones."""
    from workloads import WORKLOADS, custom, generate
    act = WORKLOADS["act16k"]
    shape = dict(B=act.B, Hq=act.Hq, Hkv=act.Hkv, S=act.S, Dqk=act.Dqk, Dv=act.Dv, scale_block=act.scale_block)
    sets = [("gaussian", custom(**shape, wid=960), False), ("activation", act, False),
            ("activation_hadamard", act, True), ("rising", custom(**shape, dist="rising", wid=961), False)]
    dev = torch.device("cuda:0")
    rec = {"shape": f"B={act.B} Hq={act.Hq} Hkv={act.Hkv} S={act.S} D={act.Dqk}", "settle_s": 1.5,
           "window_s": window_s}
    o = torch.empty((act.B, act.Hq, act.S, act.Dv), dtype=torch.bfloat16, device=dev)
    for name, w, had in sets:
        q, k, v = generate(w, seed=0)
        qc, qs = zy.quantize_fp8(torch.from_numpy(q).to(dev), w.scale_block, had)
        kc, ks = zy.quantize_fp8(torch.from_numpy(k).to(dev), w.scale_block, had)
        vc, vs = zy.quantize_fp8(torch.from_numpy(v).to(dev), w.scale_block, False)
        del q, k, v
        for lean in ((False, True) if name in ("gaussian", "activation_hadamard") else (False,)):
            key = name + ("_fp8_lean" if lean else "_fp8")
            r = sustained(tel, lambda: zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, w.scale_block, w.softmax_scale, o=o,
                                                       lean=lean), w.flops, PEAK_FP8, 1.5, window_s, stream, torch)
            rec[key] = r
            print(f"[bench] sustained 16K {key}: {r['ms']:.3f} ms, {r['frac'] * 100:.1f}% of peak, clock "
                  f"{r['gfxclk_mhz_median']} MHz, power {r.get('socket_power_w')} W, "
                  f"{r.get('energy_per_call_j')} J/call", file=sys.stderr, flush=True)
        del qc, kc, vc
    del o
    torch.cuda.empty_cache()
    return rec


def isa_energy(window_s, stream, torch):
    """Energy per instruction class (ZYFA, "Dependence of the Shader Clock on Operand
    Values": at the power limit the energy a kernel spends per call, not its cycles, sets its
    time). Each case of the probe library runs one workgroup per compute unit, one
    instruction class in a register-only loop, with launches of about 20 ms back to back for
    the sustained window. Energy per instruction over idle = (power - power of the sleeping
    case) x launch time / instructions per launch: the sleeping waves keep the chip's clocks
    and a kernel resident, so the difference is what the instructions add."""
    import ctypes
    from fp8_causal_prefill_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        sys.exit(f"{PROBE_LIB} is not built: run python -m fp8_causal_prefill_amd.build first")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.isa_energy_case_count.restype = ctypes.c_int
    lib.isa_energy_case_name.restype = ctypes.c_char_p
    lib.isa_energy_case_name.argtypes = [ctypes.c_int]
    lib.isa_energy_case_instructions.restype = ctypes.c_double
    lib.isa_energy_case_instructions.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.isa_energy_launch.restype = ctypes.c_int
    lib.isa_energy_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    tel = Telemetry(torch)
    if tel.smi is None:
        return {"error": tel.error}
    sp = ctypes.c_void_p(stream.cuda_stream)

    def launch(i, iters):
        rc = lib.isa_energy_launch(i, iters, sp)
        if rc != 0:
            raise RuntimeError(f"isa_energy_launch({i}, {iters}) returned HIP error {rc}")

    out, idle_w = {}, None
    for i in range(lib.isa_energy_case_count()):
        name = lib.isa_energy_case_name(i).decode()
        iters, ms = 64, 0.0
        while iters < (1 << 26):  # grow until one launch takes a few ms, then aim at 20 ms
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(i, iters)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            if ms >= 4.0:
                break
            iters *= 4
        iters = max(2, min(1 << 28, int(iters * 20.0 / max(ms, 1e-3))))
        n = lib.isa_energy_case_instructions(i, iters)
        rec = sustained(tel, lambda: launch(i, iters), n, 1.0, 1.0, window_s, stream, torch)
        r = {"iters": iters, "ms_per_launch": rec["ms"], "instructions_per_launch": n,
             "gfxclk_mhz": rec.get("gfxclk_mhz_median"), "socket_power_w": rec.get("socket_power_w"),
             "power_limited_fraction": rec.get("power_limited_fraction"),
             "energy_per_launch_j": rec.get("energy_per_call_j")}
        w = rec.get("socket_power_w")
        if n == 0:
            idle_w = w
        elif w is not None and idle_w is not None:
            r["pj_per_instruction_over_idle"] = (w - idle_w) * rec["ms"] * 1e-3 / n * 1e12
        out[name] = r
    return out


def timeline_summary(rec):
    """Summary of one launch's workgroup records (include/zyfa_timeline.h: an array
    [workgroups, 8] of entry, loop start, loop end and exit stamps of a 100 MHz clock, the
    HW_ID and XCC_ID registers, and the key-tile count). A compute unit is named by its XCD,
    shader engine, shader array and CU index; workgroups that ran on one compute unit one
    after another give the dispatcher's gaps (start of the next minus end of the previous).
    Times in µs from the first workgroup's entry."""
    rec = np.asarray(rec, dtype=np.int64)
    done = rec[:, 3] > 0  # workgroups that ran the loop (the others only record their entry)
    t0 = rec[:, 0].min()
    t = (rec[:, :4] - t0) * 0.01  # µs
    t[~done, 1:4] = t[~done, 0:1]
    hw, xcc = rec[:, 4], rec[:, 5]
    cu = ((xcc & 0xF) << 8) | (((hw >> 13) & 7) << 5) | (((hw >> 12) & 1) << 4) | ((hw >> 8) & 0xF)
    span = float(t[:, 3].max())
    pro, loop, epi = t[done, 1] - t[done, 0], t[done, 2] - t[done, 1], t[done, 3] - t[done, 2]
    tiles = rec[done, 6]
    gaps, ends, busy, xcd_of = [], [], [], []
    for c in np.unique(cu):
        idx = np.where(cu == c)[0]
        order = idx[np.argsort(t[idx, 0])]
        s0, s3 = t[order, 0], t[order, 3]
        g = s0[1:] - s3[:-1]
        gaps.extend(g[g >= 0].tolist())  # (overlapping workgroups on one unit give no gap)
        ends.append(float(s3.max()))
        busy.append(float((s3 - s0).sum()))
        xcd_of.append(int(c) >> 8)
    ends, busy, xcd_of = np.array(ends), np.array(busy), np.array(xcd_of)
    gaps = np.array(gaps) if gaps else np.zeros(1)
    unit_time = float(busy.sum() + gaps.sum())
    return {
        "workgroups": int(len(rec)), "compute_units": int(len(ends)), "span_us": span,
        "prologue_us_mean": float(pro.mean()) if done.any() else None,
        "loop_us_per_key_tile": float(loop.sum() / max(1, tiles.sum())) if done.any() else None,
        "epilogue_us_mean": float(epi.mean()) if done.any() else None,
        "gap_us_mean": float(gaps.mean()),
        "transition_share": float((pro.sum() + epi.sum() + gaps.sum()) / unit_time) if unit_time > 0 else None,
        "unit_busy_us_mean": float(busy.mean()), "unit_end_us_min": float(ends.min()), "unit_end_us_max": float(ends.max()),
        "tail_idle_share": float(1.0 - ends.mean() / span) if span > 0 else None,
        "xcd_end_us": [float(ends[xcd_of == x].max()) for x in sorted(set(xcd_of.tolist()))],
        "xcd_busy_us_mean": [float(busy[xcd_of == x].mean()) for x in sorted(set(xcd_of.tolist()))],
    }


def timeline(workload_name, stream, torch):
    """One launch of each prefill kernel (FP8 exact, FP8 lean, BF16) of the workload from the
    timeline build, after ten unrecorded ones, and the summary of its workgroup records."""
    import ctypes
    from fp8_causal_prefill_amd.build import TIMELINE_LIB
    from workloads import WORKLOADS, generate
    if not os.path.exists(TIMELINE_LIB):
        sys.exit(f"{TIMELINE_LIB} is not built: run python -m fp8_causal_prefill_amd.build first")
    lib = ctypes.CDLL(TIMELINE_LIB)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.zyfa_quantize_fp8.argtypes = [vp, i32, vp, vp] + [i32] * 6 + [vp]
    for fn in ("zyfa_attn_fwd_fp8", "zyfa_attn_fwd_fp8_lean"):
        getattr(lib, fn).argtypes = [vp] * 6 + [i32, vp, vp] + [i32] * 6 + [f32, vp]
    lib.zyfa_attn_fwd_bf16.argtypes = [vp] * 5 + [i32] * 6 + [f32, vp]
    lib.zyfa_timeline_clear.argtypes = [vp]
    lib.zyfa_timeline_read.argtypes = [vp, ctypes.c_longlong]
    w = WORKLOADS[workload_name]
    q, k, v = generate(w, seed=0)
    dev = torch.device("cuda:0")
    sp = ctypes.c_void_p(stream.cuda_stream)

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} returned {rc}")

    def quant(x, H):
        xd = torch.from_numpy(x).to(dev)
        nb = (w.S + w.scale_block - 1) // w.scale_block
        codes = torch.empty(xd.shape, dtype=torch.uint8, device=dev)
        scales = torch.empty((w.B, H, nb), dtype=torch.float32, device=dev)
        ok(lib.zyfa_quantize_fp8(xd.data_ptr(), 0, codes.data_ptr(), scales.data_ptr(), w.B, H, w.S, xd.shape[3],
                                 w.scale_block, 0, sp), "zyfa_quantize_fp8")
        return codes, scales, xd.bfloat16()

    (qc, qs, qb), (kc, ks, kb), (vc, vs, vb) = quant(q, w.Hq), quant(k, w.Hkv), quant(v, w.Hkv)
    o = torch.empty((w.B, w.Hq, w.S, w.Dv), dtype=torch.bfloat16, device=dev)
    shape = (w.B, w.Hq, w.Hkv, w.S, w.Dqk, w.Dv)
    calls = {
        "fp8": lambda: lib.zyfa_attn_fwd_fp8(qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), qs.data_ptr(), ks.data_ptr(),
                                             vs.data_ptr(), w.scale_block, o.data_ptr(), None, *shape,
                                             w.softmax_scale, sp),
        "fp8_lean": lambda: lib.zyfa_attn_fwd_fp8_lean(qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), qs.data_ptr(),
                                                       ks.data_ptr(), vs.data_ptr(), w.scale_block, o.data_ptr(), None,
                                                       *shape, w.softmax_scale, sp),
        "bf16": lambda: lib.zyfa_attn_fwd_bf16(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(), o.data_ptr(), None, *shape,
                                               w.softmax_scale, sp),
    }
    n_wg = w.B * w.Hq * ((w.S + 255) // 256)
    out = {"workload": workload_name, "workgroups": n_wg}
    if n_wg > 65536:
        out["note"] = "records cover the first 65536 workgroups"
        n_wg = 65536
    for name, fn in calls.items():
        for _ in range(10):
            ok(fn(), name)
        ok(lib.zyfa_timeline_clear(sp), "zyfa_timeline_clear")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ok(fn(), name)
        e1.record(stream)
        torch.cuda.synchronize()
        rec = np.zeros((n_wg, 8), dtype=np.uint64)
        ok(lib.zyfa_timeline_read(rec.ctypes.data, n_wg), "zyfa_timeline_read")
        out[name] = dict(kernel_ms=e0.elapsed_time(e1), **timeline_summary(rec))
    return out


def operand_zeros(window_s, stream, torch, zy):
    """The headline kernels on the headline shape (B=1, Hq=32, Hkv=8, S=32768, D=128) with
    one operand tensor, or all three, set to zero and the instruction stream unchanged
    (ZYFA, "Dependence of the Shader Clock on Operand Values"): each kernel runs back to back
    under the same telemetry as ``sustained``, and its time, clock, power and energy per call
    show how much of the power budget the matrix cores' operand bits take. Zero FP8 codes
    keep their scales; zero BF16 inputs are bfloat16 zeros."""
    from workloads import WORKLOADS, generate
    w = WORKLOADS["gqa32k"]
    dev = torch.device("cuda:0")
    tel = Telemetry(torch)
    if tel.smi is None:
        return {"error": tel.error}
    q, k, v = generate(w, seed=0)
    blk, tau = w.scale_block, w.softmax_scale
    f8 = [zy.quantize_fp8(torch.from_numpy(x).to(dev), blk) for x in (q, k, v)]
    b16 = [torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v)]
    del q, k, v
    o = torch.empty((w.B, w.Hq, w.S, w.Dv), dtype=torch.bfloat16, device=dev)
    rec = {"shape": f"B={w.B} Hq={w.Hq} Hkv={w.Hkv} S={w.S} D={w.Dqk}", "settle_s": 1.5, "window_s": window_s}
    for zero in ("none", "q", "k", "v", "qkv"):
        codes = [torch.zeros_like(c) if n in zero else c for n, (c, _) in zip("qkv", f8)]
        scales = [s for _, s in f8]
        bf = [torch.zeros_like(x) if n in zero else x for n, x in zip("qkv", b16)]
        kernels = [("fp8", lambda: zy.attn_fwd_fp8(*codes, *scales, blk, tau, o=o), PEAK_FP8),
                   ("fp8_lean", lambda: zy.attn_fwd_fp8(*codes, *scales, blk, tau, o=o, lean=True), PEAK_FP8),
                   ("bf16", lambda: zy.attn_fwd_bf16(*bf, tau, o=o), PEAK_BF16)]
        for name, fn, peak in kernels:
            r = sustained(tel, fn, w.flops, peak, 1.5, window_s, stream, torch)
            rec[f"{name}_zero_{zero}"] = r
            print(f"[bench] zero {zero} {name}: {r['ms']:.3f} ms, clock {r['gfxclk_mhz_median']} MHz, power "
                  f"{r.get('socket_power_w')} W, {r.get('energy_per_call_j')} J/call", file=sys.stderr, flush=True)
        del codes, bf
    return rec


def range_paths(w, qc, kc, vc, qs, ks, vs, steps, warmup, stream, torch, zy):
    """The range entry points at the benchmark shape (FP8, exact probabilities): the second
    half of the sequence as one chunk of query rows against its causal prefix (chunked
    prefill), and the keys split into two windows whose partial results zyfa_attn_merge
    combines (split-KV). Times from HIP events on the launch stream."""
    S, blk, tau = w.S, w.scale_block, w.softmax_scale
    half = (S // 2) // blk * blk
    dev = qc.device
    per_row_flops = 2.0 * (w.Dqk + w.Dv) * w.B * w.Hq
    # chunk: rows half .. S-1, each row i sees i + 1 keys (S^2/2 convention: (S^2 - half^2) / 2)
    qc2, qs2 = qc[:, :, half:].contiguous(), qs[:, :, half // blk:].contiguous()
    oc = torch.empty((w.B, w.Hq, S - half, w.Dv), dtype=torch.bfloat16, device=dev)
    ms, _ = time_kernel(lambda: zy.attn_fwd_fp8_range(qc2, kc, vc, qs2, ks, vs, blk, half, 0, S, tau, o=oc),
                        steps, warmup, stream, torch)
    chunk_flops = per_row_flops * (S * S - half * half) / 2
    rec = {"chunk": {"q_offset": half, "rows": S - half, "keys": S, "ms": ms, "tflops": chunk_flops / ms / 1e9,
                     "frac_of_fp8_peak": chunk_flops / ms / 1e9 / PEAK_FP8}}
    # split-KV: windows [0, half) and [half, S) over all rows, then the merge
    o_parts = torch.empty((2, w.B, w.Hq, S, w.Dv), dtype=torch.bfloat16, device=dev)
    l_parts = torch.empty((2, w.B, w.Hq, S), dtype=torch.float32, device=dev)
    om = torch.empty((w.B, w.Hq, S, w.Dv), dtype=torch.bfloat16, device=dev)
    lm = torch.empty((w.B, w.Hq, S), dtype=torch.float32, device=dev)
    part_ms = []
    for i, (lo, hi) in enumerate(((0, half), (half, S))):
        ms, _ = time_kernel(lambda: zy.attn_fwd_fp8_range(qc, kc, vc, qs, ks, vs, blk, 0, lo, hi, tau, o=o_parts[i],
                                                          lse=l_parts[i]), steps, warmup, stream, torch)
        part_ms.append(ms)
    merge_ms, _ = time_kernel(lambda: zy.attn_merge(o_parts, l_parts, o=om, lse=lm), steps, warmup, stream, torch)
    rows = w.B * w.Hq * S
    merge_bytes = 3 * rows * (2 * w.Dv + 4)  # read two parts (O and LSE), write one
    rec["split_kv"] = {"windows": [[0, half], [half, S]], "parts_ms": part_ms, "merge_ms": merge_ms,
                       "total_ms": sum(part_ms) + merge_ms,
                       "tflops": w.flops / (sum(part_ms) + merge_ms) / 1e9,
                       "merge_roofline": {"bound": "hbm", "achieved": merge_bytes / merge_ms / 1e6, "peak": PEAK_HBM_GBS,
                                          "unit": "GB/s", "frac": merge_bytes / merge_ms / 1e6 / PEAK_HBM_GBS,
                                          "bytes_per_launch": merge_bytes}}
    print(f"[bench] range: chunk {rec['chunk']['ms']:.3f} ms, split-KV parts {part_ms[0]:.3f} + {part_ms[1]:.3f} ms, "
          f"merge {merge_ms:.3f} ms ({merge_bytes / merge_ms / 1e6:.0f} GB/s)", file=sys.stderr, flush=True)
    del o_parts, l_parts, om, lm, oc, qc2
    return rec


VARLEN_LENGTHS = (16384, 8192, 4096, 2048, 1024, 512, 256, 256)


def varlen_batch(w, qc, kc, vc, qs, ks, vs, steps, warmup, stream, torch, zy):
    """The benchmark's tensors read as one packed batch of sequences of different lengths
    (the varlen entry point, FP8 exact): [H, T, D] with T = S, split into VARLEN_LENGTHS
    (which sum to 32768). FLOPs: 2 (Dqk + Dv) Hq L^2 / 2 per sequence of length L."""
    lengths = VARLEN_LENGTHS
    if sum(lengths) != w.S or w.B != 1:
        return None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=qc.device)
    o = torch.empty((w.Hq, w.S, w.Dv), dtype=torch.bfloat16, device=qc.device)
    args = (qc[0], kc[0], vc[0], qs[0], ks[0], vs[0], w.scale_block, cu, max(lengths), w.softmax_scale)
    ms, med = time_kernel(lambda: zy.attn_fwd_fp8_varlen(*args, o=o), steps, warmup, stream, torch)
    flops = sum(2.0 * (w.Dqk + w.Dv) * w.Hq * n * n / 2 for n in lengths)
    print(f"[bench] varlen batch {lengths}: {ms:.3f} ms", file=sys.stderr, flush=True)
    return {"lengths": list(lengths), "heads": f"Hq={w.Hq} Hkv={w.Hkv} D={w.Dqk}", "ms": ms, "ms_median": med,
            "tflops": flops / ms / 1e9, "frac_of_fp8_peak": flops / ms / 1e9 / PEAK_FP8}


PAGE_SIZE = 128


def paged_cache(w, kc, vc, ks, vs, torch):
    """The benchmark's FP8 keys and values ([1, Hkv, S, D] codes, [1, Hkv, S / block] scales)
    moved into a paged cache of PAGE_SIZE-token pages in a seeded random page order.
    Returns (k pages, v pages, k scales, v scales, block table [1, S / PAGE_SIZE] int32)."""
    from workloads import page_table
    S, P, dev = w.S, PAGE_SIZE, kc.device
    table, num_pages = page_table([S], P, seed=0)
    bt = torch.from_numpy(table).to(dev)
    idx = bt[0].long()

    def to_pages(x, rows):  # [1, H, S', ...] -> [num_pages, H, rows per page, ...]
        pages = x[0].reshape(x.shape[1], S // P, rows, *x.shape[3:]).transpose(0, 1)
        cache = torch.zeros((num_pages, *pages.shape[1:]), dtype=x.dtype, device=dev)
        cache[idx] = pages
        return cache

    blk = w.scale_block
    return to_pages(kc, P), to_pages(vc, P), to_pages(ks, P // blk), to_pages(vs, P // blk), bt


def paged_prefill(w, qc, kc, vc, qs, ks, vs, steps, warmup, stream, torch, zy):
    """The paged entry point (FP8 exact) on the benchmark's keys and values in a shuffled
    page cache (paged_cache): the whole sequence as one chunk (the plain call's work,
    through the block table) and its second half as a chunk after a cached prefix of S / 2
    tokens (the range chunk's work); and the whole-sequence call's median time over the
    plain call's on the same keys and values, the two timed in alternation."""
    if w.B != 1 or w.S % PAGE_SIZE != 0:
        return None
    S, blk, dev = w.S, w.scale_block, qc.device
    kp, vp, ksp, vsp, bt = paged_cache(w, kc, vc, ks, vs, torch)
    o = torch.empty((w.Hq, S, w.Dv), dtype=torch.bfloat16, device=dev)
    kvl = torch.tensor([S], dtype=torch.int32, device=dev)
    rec = {"page_size": PAGE_SIZE, "num_pages": kp.shape[0], "order": "seeded random permutation"}
    half = (S // 2) // blk * blk
    calls = {}
    for name, a, flops in (("whole", 0, w.flops),
                           ("chunk", half, 2.0 * (w.Dqk + w.Dv) * w.Hq * (S * S - half * half) / 2)):
        cu = torch.tensor([0, S - a], dtype=torch.int32, device=dev)
        qa, qsa = qc[0, :, a:].contiguous(), qs[0, :, a // blk:].contiguous()
        oa = o[:, :S - a] if a == 0 else torch.empty((w.Hq, S - a, w.Dv), dtype=torch.bfloat16, device=dev)
        calls[name] = lambda qa=qa, qsa=qsa, oa=oa, cu=cu, a=a: zy.attn_fwd_fp8_paged(
            qa, kp, vp, qsa, ksp, vsp, blk, cu, kvl, bt, S - a, w.softmax_scale, o=oa)
        ms, med = time_kernel(calls[name], steps, warmup, stream, torch)
        rec[name] = {"rows": S - a, "kv_len": S, "ms": ms, "ms_median": med, "tflops": flops / ms / 1e9,
                     "frac_of_fp8_peak": flops / ms / 1e9 / PEAK_FP8}
    # the layout's cost on equal terms: the whole-sequence paged call and the plain call on
    # the same keys and values, timed in alternation (the plain call's time in the headline
    # measurement comes from another point of the run, at another clock)
    oc = torch.empty((w.B, w.Hq, S, w.Dv), dtype=torch.bfloat16, device=dev)
    plain = lambda: zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, w.softmax_scale, o=oc)
    tp, tc = [], []
    for _ in range(3):
        tp.append(time_kernel(calls["whole"], steps, 2, stream, torch)[1])
        tc.append(time_kernel(plain, steps, 2, stream, torch)[1])
    rec["whole_over_plain"] = float(np.median(tp) / np.median(tc))
    del oc
    print(f"[bench] paged: whole {rec['whole']['ms']:.3f} ms, chunk {rec['chunk']['ms']:.3f} ms; "
          f"whole over the plain call, timed alternately: {rec['whole_over_plain']:.3f}", file=sys.stderr, flush=True)
    del kp, vp, ksp, vsp, o
    return rec


DECODE_BATCH = 8


def decode_setup(w, kc, vc, ks, vs, torch, zy, seed=1):
    """Decode inputs at the benchmark's heads: DECODE_BATCH sequences of S tokens each, every
    one holding the benchmark's keys and values in its own PAGE_SIZE-token pages of one
    shared cache (seeded random page order), and one new query per sequence and head
    (seeded Gaussian). FP8 (ks, vs given): kc, vc are codes, the query is quantized with
    one scale per KV group; BF16 (ks = vs = None): kc, vc are bfloat16. Returns (q [B, Hq,
    D], q scales or None, k cache, v cache, k scales or None, v scales or None, kv_lens,
    block table)."""
    from workloads import custom, generate, page_table
    B, S, P, blk, dev = DECODE_BATCH, w.S, PAGE_SIZE, w.scale_block, kc.device
    table, num_pages = page_table([S] * B, P, seed=seed)
    bt = torch.from_numpy(table).to(dev)

    def to_pages(x, rows):  # [1, H, S', ...] -> [num_pages, H, rows per page, ...], every sequence a copy
        pages = x[0].reshape(x.shape[1], S // P, rows, *x.shape[3:]).transpose(0, 1)
        cache = torch.zeros((num_pages, *pages.shape[1:]), dtype=x.dtype, device=dev)
        for i in range(B):
            cache[bt[i].long()] = pages
        return cache

    g = w.Hq // w.Hkv
    q, _, _ = generate(custom(1, B, B, w.Hq, w.Dqk, w.Dv, wid=950), seed=seed)
    qd = torch.from_numpy(q[0]).to(dev).reshape(B, w.Hkv, g, w.Dqk)
    kvl = torch.full((B,), S, dtype=torch.int32, device=dev)
    if ks is None:
        return (qd.reshape(B, w.Hq, w.Dqk).to(torch.bfloat16), None, to_pages(kc, P), to_pages(vc, P), None, None,
                kvl, bt)
    qc, qs = zy.quantize_fp8(qd, blk)
    return (qc.reshape(B, w.Hq, w.Dqk), qs, to_pages(kc, P), to_pages(vc, P), to_pages(ks, P // blk),
            to_pages(vs, P // blk), kvl, bt)


def decode_batch(w, kc, vc, ks, vs, kd, vd, steps, warmup, stream, torch, zy):
    """The decode entry points on decode_setup's batch, FP8 exact (kc, vc, ks, vs) and BF16
    (kd, vd as bfloat16): one call is the split attention kernel plus the merge.
    HBM-bound: algorithmic bytes per call are the cached keys and values (codes and
    scales) of every sequence, the queries, the partial results (written and read once)
    and the output."""
    if w.B != 1 or w.S % PAGE_SIZE != 0:
        return None
    qc, qs, kp, vp, ksp, vsp, kvl, bt = decode_setup(w, kc, vc, ks, vs, torch, zy)
    B, S, blk = DECODE_BATCH, w.S, w.scale_block
    split = zy.decode_split_keys(B, w.Hkv, S)
    o = torch.empty((B, w.Hq, w.Dv), dtype=torch.bfloat16, device=qc.device)
    ms, med = time_kernel(lambda: zy.attn_decode_fp8_paged(qc, kp, vp, qs, ksp, vsp, blk, kvl, bt, S,
                                                            w.softmax_scale, split_keys=split, o=o),
                          steps, warmup, stream, torch)
    n_splits = -(-S // split)
    kv_bytes = B * w.Hkv * S * (w.Dqk + w.Dv) + 2 * B * w.Hkv * (S // blk) * 4
    part_bytes = 2 * n_splits * B * w.Hq * (2 * w.Dv + 4)
    total = kv_bytes + part_bytes + B * w.Hq * (w.Dqk + 2 * w.Dv)
    print(f"[bench] decode B={B} x {S} keys: {ms * 1e3:.1f} us ({total / ms / 1e6:.0f} GB/s)", file=sys.stderr,
          flush=True)
    # The same call captured in a HIP graph and replayed back to back (Inference Wave 2,
    # "Methodology and Limitations": kernel timings under graph capture and replay). The
    # allocation-free entry point is the one a capturing caller uses: its splits' partial
    # results go to the library's scratch array.
    o_eager = o.clone()
    try:
        def call():
            zy.attn_decode_fp8_paged_noalloc(qc, kp, vp, qs, ksp, vsp, blk, kvl, bt, S, o,
                                             softmax_scale=w.softmax_scale, split_keys=split)

        call()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        gms = e0.elapsed_time(e1) / steps
        graph = {"entry_point": "zyfa_attn_decode_fp8_paged_noalloc", "replays": steps, "ms": gms,
                 "output_equals_eager_call": bool(torch.equal(o, o_eager)),
                 "achieved_gbs": total / gms / 1e6, "frac_of_hbm": total / gms / 1e6 / PEAK_HBM_GBS}
        print(f"[bench] decode as graph replays: {gms * 1e3:.1f} us ({total / gms / 1e6:.0f} GB/s)", file=sys.stderr,
              flush=True)
        del g
    except Exception as e:  # recorded, not fatal: the eager figures above stand
        graph = {"error": repr(e)}
    del kp, vp, ksp, vsp, qc
    rec = {"batch": B, "kv_len": S, "heads": f"Hq={w.Hq} Hkv={w.Hkv} D={w.Dqk}", "page_size": PAGE_SIZE,
           "split_keys": split, "n_splits": n_splits, "ms": ms, "ms_median": med,
           "roofline": {"bound": "hbm", "achieved": total / ms / 1e6, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": total / ms / 1e6 / PEAK_HBM_GBS, "bytes_per_call": total,
                        "kv_bytes": kv_bytes},
           "graph": graph}
    # BF16: the same batch in bfloat16 (twice the cache bytes, no scales)
    qb, _, kpb, vpb, _, _, kvl, bt = decode_setup(w, kd.to(torch.bfloat16), vd.to(torch.bfloat16), None, None,
                                                   torch, zy)
    split_b = zy.decode_split_keys(B, w.Hkv, S, 256)  # eight-wave workgroups: one per compute unit
    ms_b, med_b = time_kernel(lambda: zy.attn_decode_bf16_paged(qb, kpb, vpb, kvl, bt, S, w.softmax_scale,
                                                                 split_keys=split_b, o=o), steps, warmup, stream, torch)
    n_splits_b = -(-S // split_b)
    total_b = (2 * B * w.Hkv * S * (w.Dqk + w.Dv) + 2 * n_splits_b * B * w.Hq * (2 * w.Dv + 4)
               + B * w.Hq * (2 * w.Dqk + 2 * w.Dv))
    print(f"[bench] decode bf16: {ms_b * 1e3:.1f} us ({total_b / ms_b / 1e6:.0f} GB/s)", file=sys.stderr, flush=True)
    rec["bf16"] = {"split_keys": split_b, "ms": ms_b, "ms_median": med_b, "achieved_gbs": total_b / ms_b / 1e6,
                   "frac_of_hbm": total_b / ms_b / 1e6 / PEAK_HBM_GBS, "bytes_per_call": total_b}
    del kpb, vpb
    return rec


ERROR_HEADS = (0, 13)  # query heads whose sampled rows give the activation-like error figures
ERROR_ROWS = 256


def other_workloads(names, steps, warmup, torch, zy):
    """Kernel throughput on the other benchmark shapes (4K MHA, 32K MLA, 16K activation-like
    with and without the Hadamard rotation of Q and K): FP8 exact and lean, and BF16.
    Reported from the median launch time (these shorter runs see occasional outliers).
    For the activation-like shape also returns, per rotation setting, what the CPU leg needs
    for its error figures: the float32 inputs, the codes and scales the kernel read and the
    kernel's outputs, for ERROR_ROWS sampled rows of the ERROR_HEADS query heads."""
    from workloads import WORKLOADS, generate, sample_rows
    out, samples = {}, {}
    stream = torch.cuda.current_stream()
    for name in names:
        w = WORKLOADS[name]
        q, k, v = generate(w, seed=0)
        dev = torch.device("cuda:0")
        qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
        if w.dist == "activation":
            group = w.Hq // w.Hkv
            rows = sample_rows(w.S, ERROR_ROWS, seed=1)
            samples[name] = {"w": w, "rows": rows, "heads": ERROR_HEADS,
                             "inputs": {h: (q[0, h], k[0, h // group], v[0, h // group]) for h in ERROR_HEADS}}
        del q, k, v
        rec = {"shape": f"B={w.B} Hq={w.Hq} Hkv={w.Hkv} S={w.S} Dqk={w.Dqk} Dv={w.Dv}", "flops": w.flops}
        # the Q quantization pass, without and with the Hadamard rotation (HBM-bound: 4 bytes
        # read and 1 written per element, plus one scale per block)
        qbytes = qd.numel() * 5 + qd.numel() // (w.Dqk * w.scale_block) * 4
        # (into preallocated outputs: at 4K tokens the pass takes about as long as the
        # binding's allocations would, and the launches must not wait for the host)
        qcode = torch.empty(qd.shape, dtype=torch.uint8, device=dev)
        qscale = torch.empty((w.B, w.Hq, -(-w.S // w.scale_block)), dtype=torch.float32, device=dev)
        for had in (False, True):
            ms, med = time_kernel(lambda: zy.quantize_fp8(qd, w.scale_block, had, qcode, qscale), steps, warmup,
                                  stream, torch)
            rec["quantize_q" + ("_hadamard" if had else "")] = {"ms": med, "gbs": qbytes / med / 1e6,
                                                                  "frac_of_hbm": qbytes / med / 1e6 / PEAK_HBM_GBS}
        for had in ((False, True) if w.dist == "activation" else (False,)):
            qc, qs = zy.quantize_fp8(qd, w.scale_block, had)
            kc, ks = zy.quantize_fp8(kd, w.scale_block, had)
            vc, vs = zy.quantize_fp8(vd, w.scale_block, False)
            o = torch.empty((w.B, w.Hq, w.S, w.Dv), dtype=torch.bfloat16, device=dev)
            tag = "_hadamard" if had else ""
            for mode in ("fp8", "fp8_lean"):
                lean = mode == "fp8_lean"
                ms, med = time_kernel(lambda: zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, w.scale_block, w.softmax_scale,
                                                              o=o, lean=lean), steps, warmup, stream, torch)
                rec[mode + tag] = {"ms_mean": ms, "ms": med, "tflops": w.flops / med / 1e9,
                                   "frac_of_fp8_peak": w.flops / med / 1e9 / PEAK_FP8}
                if name in samples:
                    sm = samples[name].setdefault(had, {})
                    idx = torch.from_numpy(samples[name]["rows"]).to(dev)
                    for h in ERROR_HEADS:
                        g = h // (w.Hq // w.Hkv)
                        sm.setdefault(h, {"codes": tuple(t[0, hh].cpu().numpy() for t, hh in
                                                         ((qc, h), (qs, h), (kc, g), (ks, g), (vc, g), (vs, g)))})
                        sm[h][mode] = o[0, h].index_select(0, idx).float().cpu().numpy().astype(np.float64)
            del qc, kc, vc
        qb, kb, vb = qd.to(torch.bfloat16), kd.to(torch.bfloat16), vd.to(torch.bfloat16)
        ob = torch.empty((w.B, w.Hq, w.S, w.Dv), dtype=torch.bfloat16, device=dev)
        ms, med = time_kernel(lambda: zy.attn_fwd_bf16(qb, kb, vb, w.softmax_scale, o=ob), steps, warmup, stream, torch)
        rec["bf16"] = {"ms_mean": ms, "ms": med, "tflops": w.flops / med / 1e9,
                       "frac_of_bf16_peak": w.flops / med / 1e9 / PEAK_BF16}
        out[name] = rec
        print(f"[bench] {name}: fp8 {rec['fp8']['ms']:.3f} ms, lean {rec['fp8_lean']['ms']:.3f} ms, "
              f"bf16 {rec['bf16']['ms']:.3f} ms", file=sys.stderr, flush=True)
        del qd, kd, vd, qb, kb, vb, o, ob, qcode, qscale
        torch.cuda.empty_cache()
    return out, samples


def activation_errors(sample):
    """Error figures of the activation-like workload (ZYFA, "FP8 Error in Full-Model
    Inference": the rotation of Q and K roughly halves the error that input quantization
    adds), from the sampled rows other_workloads kept, per rotation setting:

    * kernel_rel_l2_fp8 / _lean: the kernel against the fp64 oracle on the codes and scales
      it read (the parity figure);
    * input_quantization_rel_l2: the oracle on those dequantized inputs against fp64
      attention on the unquantized float32 inputs (the rotation is orthonormal, so the
      unrotated inputs give the same scores);
    * end_to_end_rel_l2_fp8 / _lean: the kernel against attention on the unquantized inputs.

    Runs the oracle, so it belongs to the CPU leg."""
    from oracle import causal_attention, dequantize_blocks
    w, rows, heads = sample["w"], sample["rows"], sample["heads"]
    blk = w.scale_block
    rel = lambda a, b: float(np.sqrt(np.sum((a - b) ** 2) / np.sum(b ** 2)))
    exact = {}
    for h in heads:
        qh, kh, vh = sample["inputs"][h]
        exact[h] = causal_attention(qh[None, None], kh[None, None], vh[None, None], w.softmax_scale, rows=rows)[0][0, 0]
    out = {"rows_per_head": len(rows), "heads": list(heads)}
    for had in (False, True):
        sm = sample.get(had)
        if sm is None:
            continue
        refs, got = {}, {"fp8": {}, "fp8_lean": {}}
        for h in heads:
            qc, qs, kc, ks, vc, vs = sm[h]["codes"]
            deq = [dequantize_blocks(c[None, None], sc[None, None], blk) for c, sc in ((qc, qs), (kc, ks), (vc, vs))]
            refs[h] = causal_attention(*deq, w.softmax_scale, rows=rows)[0][0, 0]
            for mode in got:
                got[mode][h] = sm[h][mode]
        cat = lambda d: np.concatenate([d[h] for h in heads])
        ref_q, ref_x = cat(refs), cat(exact)
        out["hadamard" if had else "no_rotation"] = {
            "kernel_rel_l2_fp8": rel(cat(got["fp8"]), ref_q), "kernel_rel_l2_fp8_lean": rel(cat(got["fp8_lean"]), ref_q),
            "input_quantization_rel_l2": rel(ref_q, ref_x),
            "end_to_end_rel_l2_fp8": rel(cat(got["fp8"]), ref_x),
            "end_to_end_rel_l2_fp8_lean": rel(cat(got["fp8_lean"]), ref_x)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="gqa32k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-lean", action="store_true", help="skip the lean-probability FP8 mode")
    ap.add_argument("--no-others", action="store_true", help="skip the other workload shapes")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the FP8 kernel timed after flushes of L2 and the Infinity Cache")
    ap.add_argument("--no-range", action="store_true", help="skip the varlen, chunked-prefill, split-KV, paged and decode measurements")
    ap.add_argument("--sustain", type=float, default=4.0,
                    help="seconds of back-to-back launches per headline kernel, after 1.5 s of settling, "
                         "with clock and power telemetry (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    ap.add_argument("--operand-zeros", action="store_true",
                    help="only run the headline kernels with Q, K, V or all three zeroed, under the sustained "
                         "telemetry, and print that record as one JSON line")
    ap.add_argument("--timeline", action="store_true",
                    help="only run the workload's prefill kernels once each from the timeline build and print "
                         "the summary of their workgroup records as one JSON line")
    ap.add_argument("--isa-energy", action="store_true",
                    help="only run the probe library's instruction classes under the sustained telemetry "
                         "and print power, clock and energy per instruction as one JSON line")
    ap.add_argument("--isa-costs", action="store_true",
                    help="only run the instruction-cost probe (matrix and vector instruction cycles, "
                         "matrix/vector overlap in one wave) and print its JSON line")
    args = ap.parse_args()

    if args.isa_costs:
        from fp8_causal_prefill_amd.build import PROBE
        if not os.path.exists(PROBE):
            sys.exit(f"{PROBE} is not built: run python -m fp8_causal_prefill_amd.build first")
        r = subprocess.run([PROBE], capture_output=True, text=True, timeout=120)
        if r.returncode != 0:
            sys.exit(f"isa_cost exited with {r.returncode}: {r.stderr.strip()}")
        print(json.dumps({"isa_costs": json.loads(r.stdout), "device": "cuda:0"}))
        return

    if args.timeline:
        import torch
        stream = torch.cuda.current_stream()
        print(json.dumps({"timeline": timeline(args.workload, stream, torch), "device": "cuda:0"}))
        return

    if args.isa_energy:
        import torch
        stream = torch.cuda.current_stream()
        print(json.dumps({"isa_energy": isa_energy(max(args.sustain, 1.0), stream, torch), "device": "cuda:0"}))
        return

    if args.operand_zeros:
        import torch
        import fp8_causal_prefill_amd as zy
        stream = torch.cuda.current_stream()
        print(json.dumps({"operand_zeros": operand_zeros(max(args.sustain, 1.0), stream, torch, zy)}))
        return

    if args.copy_calibration:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "launches": 5}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_causal_prefill_amd as zy
    from workloads import WORKLOADS, generate

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} S={w.S} Dqk={w.Dqk} Dv={w.Dv}", file=sys.stderr,
          flush=True)
    q, k, v = generate(w, seed=0)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    blk = w.scale_block
    scale = w.softmax_scale
    flops = w.flops

    # ---------------- FP8: quantize + attention ----------------
    qc = torch.empty(qd.shape, dtype=torch.uint8, device=dev)
    kc = torch.empty(kd.shape, dtype=torch.uint8, device=dev)
    vc = torch.empty(vd.shape, dtype=torch.uint8, device=dev)
    nb = (w.S + blk - 1) // blk
    qs = torch.empty((w.B, w.Hq, nb), dtype=torch.float32, device=dev)
    ks = torch.empty((w.B, w.Hkv, nb), dtype=torch.float32, device=dev)
    vs = torch.empty((w.B, w.Hkv, nb), dtype=torch.float32, device=dev)
    o8 = torch.empty((w.B, w.Hq, w.S, w.Dv), dtype=torch.bfloat16, device=dev)
    o8l = torch.empty_like(o8)

    stream = torch.cuda.current_stream()
    ev = []

    def fp8_step(record=False):
        zy.quantize_fp8(qd, blk, False, qc, qs)
        zy.quantize_fp8(kd, blk, False, kc, ks)
        zy.quantize_fp8(vd, blk, False, vc, vs)
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, scale, o=o8)
            e1.record(stream)
            ev.append((e0, e1))
        else:
            zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, scale, o=o8)

    for _ in range(args.warmup):
        fp8_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fp8_step(record=True)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    attn_s = float(np.mean(attn_ms)) / 1e3
    attn_med_s = float(np.median(attn_ms)) / 1e3
    print(f"[bench] fp8 step {step_s * 1e3:.3f} ms, attention kernel mean {attn_s * 1e3:.3f} ms "
          f"(median {attn_med_s * 1e3:.3f})", file=sys.stderr, flush=True)

    # ---------------- FP8 attention, lean probabilities (opt-in mode) ----------------
    lean = None
    if not args.no_lean:
        evl = []
        for _ in range(max(args.warmup // 2, 1)):
            zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, scale, o=o8l, lean=True)
        torch.cuda.synchronize()
        lsteps = max(args.steps // 2, 1)
        for _ in range(lsteps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, scale, o=o8l, lean=True)
            e1.record(stream)
            evl.append((e0, e1))
        torch.cuda.synchronize()
        lms = [a.elapsed_time(b) for a, b in evl]
        l_s = float(np.mean(lms)) / 1e3
        print(f"[bench] fp8 lean attention kernel mean {l_s * 1e3:.3f} ms", file=sys.stderr, flush=True)
        lean = {"entry_point": "zyfa_attn_fwd_fp8_lean", "tflops": flops / l_s / 1e12, "ms": l_s * 1e3,
                "ms_median": float(np.median(lms)), "frac_of_fp8_peak": flops / l_s / 1e12 / PEAK_FP8,
                "steps": lsteps}

    # ---------------- BF16 attention ----------------
    bf16 = None
    if not args.no_bf16:
        qb, kb, vb = qd.to(torch.bfloat16), kd.to(torch.bfloat16), vd.to(torch.bfloat16)
        ob = torch.empty((w.B, w.Hq, w.S, w.Dv), dtype=torch.bfloat16, device=dev)
        evb = []

        def bf16_step():
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            zy.attn_fwd_bf16(qb, kb, vb, scale, o=ob)
            e1.record(stream)
            evb.append((e0, e1))

        for _ in range(max(args.warmup // 2, 1)):
            zy.attn_fwd_bf16(qb, kb, vb, scale, o=ob)
        torch.cuda.synchronize()
        bsteps = max(args.steps // 2, 1)
        t0 = time.perf_counter()
        for _ in range(bsteps):
            bf16_step()
        torch.cuda.synchronize()
        bstep_s = (time.perf_counter() - t0) / bsteps
        bms = [a.elapsed_time(b) for a, b in evb]
        b_s = float(np.mean(bms)) / 1e3
        print(f"[bench] bf16 attention kernel mean {b_s * 1e3:.3f} ms", file=sys.stderr, flush=True)
        bf16 = {"tflops": flops / b_s / 1e12, "ms": b_s * 1e3, "ms_median": float(np.median(bms)),
                "frac_of_bf16_peak": flops / b_s / 1e12 / PEAK_BF16, "frac_of_fp8_peak": flops / b_s / 1e12 / PEAK_FP8,
                "peak": PEAK_BF16, "steps": bsteps, "step_ms": bstep_s * 1e3,
                "hbm_traffic": hbm_traffic(w.name, "bf16")}

    # ---------------- sustained clocks: telemetry while each kernel runs back to back ----------------
    sustained_rec = None
    if args.sustain > 0:
        tel = Telemetry(torch)
        if tel.smi is None:
            sustained_rec = {"error": tel.error}
        else:
            sustained_rec = {"settle_s": 1.5, "window_s": args.sustain}
            kernels = [("fp8", lambda: zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, scale, o=o8), PEAK_FP8)]
            if not args.no_lean:
                kernels.append(("fp8_lean", lambda: zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, scale, o=o8l,
                                                                    lean=True), PEAK_FP8))
            if not args.no_bf16:
                kernels.append(("bf16", lambda: zy.attn_fwd_bf16(qb, kb, vb, scale, o=ob), PEAK_BF16))
            for name, fn, peak in kernels:
                sustained_rec[name] = sustained(tel, fn, flops, peak, 1.5, args.sustain, stream, torch)
                r = sustained_rec[name]
                print(f"[bench] sustained {name}: {r['ms']:.3f} ms, {r['frac'] * 100:.1f}% of peak, "
                      f"clock {r['gfxclk_mhz_median']} MHz, power {r.get('socket_power_w')} W", file=sys.stderr,
                      flush=True)
            if not args.no_others:
                sustained_rec["structured_inputs"] = structured_sustained(tel, args.sustain, stream, torch, zy)

    # ---------------- cold caches: the FP8 kernel after each flush of L2 and the Infinity Cache ----------------
    cold = None
    if not args.no_cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)  # twice the 256 MiB Infinity Cache
        evc = []
        for i in range(2 * args.steps + 2):
            flush.fill_(i & 0xFF)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, scale, o=o8)
            e1.record(stream)
            if i >= 2:
                evc.append((e0, e1))
        torch.cuda.synchronize()
        cms = [a.elapsed_time(b) for a, b in evc]
        cold = {"launches": len(cms), "flush_bytes": 512 << 20, "ms_median": float(np.median(cms)),
                "ms_mean": float(np.mean(cms)), "warm_ms_median": attn_med_s * 1e3}
        del flush
        print(f"[bench] fp8 attention after cache flushes: median {cold['ms_median']:.3f} ms over {len(cms)} launches",
              file=sys.stderr, flush=True)

    achieved = flops / attn_s / 1e12
    line = {
        "metric": "causal prefill attn TFLOPS + % of FP8 MFMA peak, S=32K D=128 (FP8 & BF16)",
        "value": flops / step_s / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: causal prefill B={w.B} Hq={w.Hq} Hkv={w.Hkv} S={w.S} Dqk={w.Dqk} "
                               f"Dv={w.Dv}, Q/K/V ~ N(0,1) float32, e4m3 scale block {blk}",
                   "step": "quantize Q,K,V (e4m3, per-block scales) + FP8 attention",
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP8, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP8, "traffic": hbm_traffic(w.name, "fp8"),
                     "kernel": "attn_fwd_kernel<FP8, 128>", "kernel_ms_mean": attn_s * 1e3,
                     "kernel_ms_median": attn_med_s * 1e3},
        "fp8_lean": lean,
        "bf16": bf16,
        "sustained": sustained_rec,
        "cold_caches": cold,
    }

    if not args.no_range:
        line["varlen"] = varlen_batch(w, qc, kc, vc, qs, ks, vs, max(args.steps // 5, 5), max(args.warmup // 10, 5),
                                      stream, torch, zy)
        line["range"] = range_paths(w, qc, kc, vc, qs, ks, vs, max(args.steps // 5, 5), max(args.warmup // 10, 5), stream,
                                    torch, zy)
        line["paged"] = paged_prefill(w, qc, kc, vc, qs, ks, vs, max(args.steps // 5, 5), max(args.warmup // 10, 5),
                                      stream, torch, zy)
        line["decode"] = decode_batch(w, kc, vc, ks, vs, kd, vd, max(args.steps // 5, 5), max(args.warmup // 10, 5),
                                      stream, torch, zy)

    if not args.no_others:
        others = [n for n in ("mha4k", "mla32k", "act16k") if n != w.name]
        line["other_workloads"], error_samples = other_workloads(others, max(args.steps // 5, 5),
                                                                 max(args.warmup // 10, 5), torch, zy)

    if not args.no_cpu:
        for name, sample in (error_samples if not args.no_others else {}).items():
            t0 = time.perf_counter()
            line["other_workloads"][name]["error"] = activation_errors(sample)
            print(f"[bench] {name} error figures ({time.perf_counter() - t0:.1f} s): "
                  f"{json.dumps(line['other_workloads'][name]['error'])}", file=sys.stderr, flush=True)
        cpu, refs = cpu_baseline(w, q, k, v)
        # the sampled heads also give a full-size parity figure for the timed configuration
        num = den = 0.0
        for hq, ref in refs.items():
            got = o8[0, hq].float().cpu().numpy().astype(np.float64)
            num += float(np.sum((got - ref) ** 2))
            den += float(np.sum(ref ** 2))
        line["cpu_baseline"] = cpu
        line["sampled_rel_l2_fp8"] = math.sqrt(num / den)
        if lean is not None:
            num = 0.0
            for hq, ref in refs.items():
                got = o8l[0, hq].float().cpu().numpy().astype(np.float64)
                num += float(np.sum((got - ref) ** 2))
            lean["sampled_rel_l2"] = math.sqrt(num / den)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
