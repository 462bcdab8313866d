"""The instruction-cost probe library (fp8_causal_prefill_amd/libisa_cost.so) without a GPU:
it loads, its case table is consistent, and its launcher rejects invalid requests before
any HIP call. `bench.py --isa-energy` reads the case names and instruction counts from it
and divides measured energy by those counts, so the counts are checked here against the
loop shapes of the probe's kernels."""

import ctypes
import os

import pytest

from fp8_causal_prefill_amd.build import PROBE, PROBE_LIB

HIP_ERROR_INVALID_VALUE = 1


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: build it with `python -m fp8_causal_prefill_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.isa_energy_case_count.restype = ctypes.c_int
    lib.isa_energy_case_name.restype = ctypes.c_char_p
    lib.isa_energy_case_name.argtypes = [ctypes.c_int]
    lib.isa_energy_case_instructions.restype = ctypes.c_double
    lib.isa_energy_case_instructions.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.isa_energy_launch.restype = ctypes.c_int
    lib.isa_energy_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


def cases(probe):
    return [probe.isa_energy_case_name(i).decode() for i in range(probe.isa_energy_case_count())]


def test_program_and_library_are_built():
    assert os.access(PROBE, os.X_OK)
    assert os.path.exists(PROBE_LIB)


def test_case_table(probe):
    names = cases(probe)
    assert len(names) == len(set(names)) >= 10
    assert names[0].startswith("idle")  # the baseline that every other case is measured against
    assert probe.isa_energy_case_name(-1) is None
    assert probe.isa_energy_case_name(len(names)) is None
    assert probe.isa_energy_case_instructions(len(names), 100) == -1.0


def test_instruction_counts_follow_the_loops(probe):
    # 256 workgroups; waves = 256 x 4 SIMDs x waves per SIMD
    by = {n: i for i, n in enumerate(cases(probe))}

    def count(prefix, iters):
        (name,) = [n for n in by if n.startswith(prefix)]
        return probe.isa_energy_case_instructions(by[name], iters)

    assert count("idle", 1000) == 0.0
    assert count("mfma 32x32x64 e4m3, random", 1000) == 256 * 4 * 1 * 1000 * 4
    assert count("mfma 32x32x16 bf16, zero", 10) == 256 * 4 * 1 * 10 * 4
    assert count("v_exp_f32", 1000) == 256 * 4 * 2 * 1000 * 64
    assert count("s_add_u32", 7) == 256 * 4 * 2 * 7 * 16
    # LDS loops take iterations in pairs and read one batch of eight ahead
    assert count("ds_read_b128", 100) == 256 * 4 * 4 * 101 * 8
    assert count("ds_read_b64_tr_b8", 101) == 256 * 4 * 4 * 103 * 8


@pytest.mark.parametrize("case,iters", [(-1, 100), (10 ** 6, 100), (0, 1), (0, -5), (0, (1 << 30) + 1)])
def test_launch_rejects_invalid_requests_on_the_host(probe, case, iters):
    assert probe.isa_energy_launch(case, iters, None) == HIP_ERROR_INVALID_VALUE
