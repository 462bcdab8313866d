"""Build libzyfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m fp8_causal_prefill_amd.build

Every source is compiled by hipcc for gfx950 only, with packed FP32 instructions
disabled, and linked into fp8_causal_prefill_amd/libzyfa.so next to this file.
The timeline build, libzyfa_timeline.so (include/zyfa_timeline.h: the same library with
per-workgroup time stamps in the prefill kernels, read by `bench.py --timeline`), is linked
next to it from a second compile of the attention kernels.
The instruction-cost probe (csrc/probes/isa_cost.hip) is built next to it twice: as the
stand-alone program fp8_causal_prefill_amd/isa_cost that `bench.py --isa-costs` runs, and
as fp8_causal_prefill_amd/libisa_cost.so, whose kernels `bench.py --isa-energy` launches
under the power telemetry.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libzyfa.so")
TIMELINE_LIB = os.path.join(HERE, "libzyfa_timeline.so")
SOURCES = ["capi.cpp", "attn_fwd.hip", "quantize.hip", "merge.hip", "scratch.hip"]
PROBE_SRC = os.path.join(CSRC, "probes", "isa_cost.hip")
PROBE = os.path.join(HERE, "isa_cost")
PROBE_LIB = os.path.join(HERE, "libisa_cost.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        # packed FP32 VALU ops are kept out of all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(HERE, "..", "include"),
    ]


def _compile(src: str, extra, tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [hipcc()] + common_flags() + list(extra) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so: harmless
    noise = "packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def _link(out: str, objs) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + list(objs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)


def build(extra_flags=(), verbose=False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, list(extra_flags), "") for s in SOURCES] + [("attn_fwd.hip", list(extra_flags) + ["-DZYFA_TIMELINE"],
                                                             "_timeline")]
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(LIB, objs[:len(SOURCES)])
    _link(TIMELINE_LIB, [objs[-1] if s == "attn_fwd.hip" else o for s, o in zip(SOURCES, objs)])
    build_probe(extra_flags)
    if verbose:
        print(f"built {LIB}, {TIMELINE_LIB}, {PROBE} and {PROBE_LIB}")
    return LIB


def build_probe(extra_flags=()) -> str:
    for out, mode in ((PROBE, []), (PROBE_LIB, ["-DISA_COST_LIB", "-shared"])):
        tmp = out + ".tmp"
        cmd = [hipcc()] + common_flags() + list(extra_flags) + mode + ["-x", "hip", PROBE_SRC, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
        os.replace(tmp, out)
    return PROBE


if __name__ == "__main__":
    build(verbose=True)
