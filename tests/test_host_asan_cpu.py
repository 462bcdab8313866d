"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

capi.cpp (argument validation, dispatch and error reporting: all the host code the library
runs before a launch) is built with g++ and -fsanitize=address,undefined (undefined
behaviour fatal) against stub launchers,
and the CPU ABI tests (tests/test_abi_cpu.py: every entry point with every class of
invalid request, and the workspace-size arithmetic; not the ones that need the Python
package with torch or a child process of their own) run against that build in a child
process with the address sanitizer's runtime preloaded. Any out-of-bounds access, use
after free, signed overflow or other undefined behaviour in the host checks (the
workspace-size arithmetic's overflow guard among them) ends the child with a report. No device code is
built or run: the stubs stand in for the kernels' launchers, which no invalid request
reaches.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp8_causal_prefill_amd")
CSRC = os.path.join(PKG, "csrc")
HIP_LIB = "/opt/rocm/lib/libamdhip64.so"

STUBS = """#include "launch.h"
namespace zyfa {
hipError_t launch_attn_fwd_fp8(const AttnArgs&, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_fwd_bf16(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_quantize_fp8(const QuantArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_merge(const MergeArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t scratch_of_stream_device(hipStream_t, void**) { return hipErrorNotSupported; }
}  // namespace zyfa
"""

CHILD = """
import ctypes, sys, types
assert hasattr(ctypes.CDLL(None), "__asan_report_load1"), "the sanitizer runtime is not loaded"
pkg = types.ModuleType("fp8_causal_prefill_amd")  # the ctypes module alone, without torch
pkg.__path__ = [{pkg!r}]
sys.modules["fp8_causal_prefill_amd"] = pkg
from fp8_causal_prefill_amd import _lib
_lib.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "--noconftest", "-p", "no:cacheprovider", {tests!r}, "-k", "not debug_env and not binding"]))
"""


def _asan_runtime():
    if shutil.which("g++") is None:
        return None
    p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_abi_host_checks_under_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(HIP_LIB):
        pytest.skip("needs g++ with libasan and the HIP runtime library")
    (tmp_path / "stubs.cpp").write_text(STUBS)
    lib = str(tmp_path / "libzyfa_asan.so")
    cmd = ["g++", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-std=c++17",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", CSRC, "-fPIC", "-shared",
           os.path.join(CSRC, "capi.cpp"), str(tmp_path / "stubs.cpp"), "-L/opt/rocm/lib", "-lamdhip64", "-o", lib]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr
    code = CHILD.format(pkg=PKG, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
