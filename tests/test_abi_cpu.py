"""The C-ABI library without a GPU: it loads, exports every entry point that
include/zyfa.h declares, and rejects invalid requests on the host before any HIP
call (fake, never-dereferenced pointers are used; no request here is valid, so no
kernel is ever launched)."""

import ctypes
import os
import re

import pytest

from fp8_causal_prefill_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "zyfa.h")

P = 0x10000   # a 16-byte-aligned fake device address (never dereferenced)
P2 = 0x20000
P3 = 0x30000
P4 = 0x40000
P5 = 0x50000
P6 = 0x60000
P7 = 0x70000
MIS = 0x10008  # misaligned


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(zyfa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"zyfa_abi_version", "zyfa_status_string", "zyfa_last_error", "zyfa_quantize_fp8",
                          "zyfa_attn_fwd_fp8", "zyfa_attn_fwd_fp8_lean", "zyfa_attn_fwd_bf16",
                          "zyfa_attn_fwd_fp8_range", "zyfa_attn_fwd_bf16_range", "zyfa_attn_merge",
                          "zyfa_attn_fwd_fp8_varlen", "zyfa_attn_fwd_bf16_varlen", "zyfa_attn_fwd_fp8_paged",
                          "zyfa_attn_fwd_bf16_paged", "zyfa_attn_decode_workspace_bytes", "zyfa_attn_decode_fp8_paged",
                          "zyfa_attn_decode_bf16_paged", "zyfa_attn_decode_fp8_paged_noalloc"}
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_strings(lib):
    assert lib.zyfa_abi_version() == 6
    assert lib.zyfa_status_string(0) == b"ZYFA_OK"
    assert lib.zyfa_status_string(1) == b"ZYFA_ERR_INVALID_ARGUMENT"
    assert lib.zyfa_status_string(2) == b"ZYFA_ERR_UNSUPPORTED"
    assert lib.zyfa_status_string(3) == b"ZYFA_ERR_LAUNCH"
    assert lib.zyfa_status_string(99) == b"ZYFA_UNKNOWN_STATUS"


def fp8(lib, q=P, k=P2, v=P3, qs=P4, ks=P5, vs=P6, blk=128, o=P7, lse=None, B=1, Hq=4, Hkv=2, S=256, Dqk=128,
        Dv=128, scale=0.088, lean=False):
    fn = lib.zyfa_attn_fwd_fp8_lean if lean else lib.zyfa_attn_fwd_fp8
    return fn(q, k, v, qs, ks, vs, blk, o, lse, B, Hq, Hkv, S, Dqk, Dv, scale, None)


def bf16(lib, q=P, k=P2, v=P3, o=P7, lse=None, B=1, Hq=4, Hkv=2, S=256, Dqk=128, Dv=128, scale=0.088):
    return lib.zyfa_attn_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, S, Dqk, Dv, scale, None)


INVALID = _lib.ERR_INVALID_ARGUMENT
UNSUPPORTED = _lib.ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(q=MIS), INVALID), (dict(o=MIS), INVALID), (dict(lse=MIS), INVALID),
    (dict(B=0), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=0), INVALID), (dict(S=0), INVALID), (dict(S=-5), INVALID),
    (dict(Hq=6, Hkv=4), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(Dqk=64, Dv=64), UNSUPPORTED), (dict(Dqk=192, Dv=192), UNSUPPORTED), (dict(Dqk=128, Dv=192), UNSUPPORTED),
    (dict(o=P), INVALID),  # output aliases q
])
def test_attention_argument_checks(lib, kw, expect):
    assert bf16(lib, **kw) == expect
    assert lib.zyfa_last_error() != b""
    assert fp8(lib, **kw) == expect
    assert fp8(lib, lean=True, **kw) == expect


@pytest.mark.parametrize("kw", [dict(qs=None), dict(ks=None), dict(vs=None), dict(vs=MIS), dict(blk=32),
                                dict(blk=0), dict(blk=256)])
def test_fp8_scale_checks(lib, kw):
    assert fp8(lib, **kw) == INVALID
    assert fp8(lib, lean=True, **kw) == INVALID


def fp8_range(lib, q=P, k=P2, v=P3, qs=P4, ks=P5, vs=P6, blk=128, o=P7, lse=None, B=1, Hq=4, Hkv=2, Sq=256, Skv=512,
              q_offset=256, k_begin=0, k_end=512, Dqk=128, Dv=128, scale=0.088, lean=0):
    return lib.zyfa_attn_fwd_fp8_range(q, k, v, qs, ks, vs, blk, o, lse, B, Hq, Hkv, Sq, Skv, q_offset, k_begin, k_end,
                                       Dqk, Dv, scale, lean, None)


def bf16_range(lib, q=P, k=P2, v=P3, o=P7, lse=None, B=1, Hq=4, Hkv=2, Sq=256, Skv=512, q_offset=256, k_begin=0,
               k_end=512, Dqk=128, Dv=128, scale=0.088):
    return lib.zyfa_attn_fwd_bf16_range(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, q_offset, k_begin, k_end, Dqk, Dv, scale,
                                        None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(o=MIS), INVALID), (dict(Sq=0), INVALID), (dict(Skv=0), INVALID),
    (dict(q_offset=-1), INVALID), (dict(q_offset=(1 << 30) - 255), INVALID),
    (dict(k_begin=-64), INVALID), (dict(k_begin=32), INVALID), (dict(k_begin=128, k_end=128), INVALID),
    (dict(k_begin=192, k_end=100), INVALID), (dict(k_end=513), INVALID), (dict(k_end=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(scale=0.0), INVALID), (dict(Dqk=64, Dv=64), UNSUPPORTED),
    (dict(o=P2), INVALID),  # output aliases k
])
def test_range_argument_checks(lib, kw, expect):
    assert bf16_range(lib, **kw) == expect
    assert lib.zyfa_last_error() != b""
    assert fp8_range(lib, **kw) == expect
    assert fp8_range(lib, lean=1, **kw) == expect


@pytest.mark.parametrize("kw", [dict(qs=None), dict(vs=MIS), dict(blk=32), dict(lean=2), dict(lean=-1)])
def test_fp8_range_scale_and_mode_checks(lib, kw):
    assert fp8_range(lib, **kw) == INVALID


def fp8_varlen(lib, q=P, k=P2, v=P3, qs=P4, ks=P5, vs=P6, blk=128, o=P7, lse=None, cu=0x80000, n=3, maxs=300,
               Hq=4, Hkv=2, T=1000, Dqk=128, Dv=128, scale=0.088, lean=0):
    return lib.zyfa_attn_fwd_fp8_varlen(q, k, v, qs, ks, vs, blk, o, lse, cu, n, maxs, Hq, Hkv, T, Dqk, Dv, scale, lean,
                                        None)


def bf16_varlen(lib, q=P, k=P2, v=P3, o=P7, lse=None, cu=0x80000, n=3, maxs=300, Hq=4, Hkv=2, T=1000, Dqk=128,
                Dv=128, scale=0.088):
    return lib.zyfa_attn_fwd_bf16_varlen(q, k, v, o, lse, cu, n, maxs, Hq, Hkv, T, Dqk, Dv, scale, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(o=MIS), INVALID), (dict(cu=None), INVALID), (dict(cu=0x80002), INVALID),
    (dict(n=0), INVALID), (dict(maxs=0), INVALID), (dict(maxs=1001), INVALID), (dict(T=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(scale=float("nan")), INVALID), (dict(Dqk=64, Dv=64), UNSUPPORTED),
    (dict(o=P), INVALID),
])
def test_varlen_argument_checks(lib, kw, expect):
    assert bf16_varlen(lib, **kw) == expect
    assert lib.zyfa_last_error() != b""
    assert fp8_varlen(lib, **kw) == expect


@pytest.mark.parametrize("kw", [dict(qs=None), dict(blk=32), dict(lean=3)])
def test_fp8_varlen_scale_and_mode_checks(lib, kw):
    assert fp8_varlen(lib, **kw) == INVALID


def fp8_paged(lib, q=P, k=P2, v=P3, qs=P4, ks=P5, vs=P6, blk=128, o=P7, lse=None, cu=0x80000, kvl=0x90000,
              bt=0xA0000, n=3, maxs=300, maxp=8, nump=30, page=128, Hq=4, Hkv=2, T=1000, Dqk=128, Dv=128,
              scale=0.088, lean=0):
    return lib.zyfa_attn_fwd_fp8_paged(q, k, v, qs, ks, vs, blk, o, lse, cu, kvl, bt, n, maxs, maxp, nump, page, Hq,
                                       Hkv, T, Dqk, Dv, scale, lean, None)


def bf16_paged(lib, q=P, k=P2, v=P3, o=P7, lse=None, cu=0x80000, kvl=0x90000, bt=0xA0000, n=3, maxs=300, maxp=8,
               nump=30, page=128, Hq=4, Hkv=2, T=1000, Dqk=128, Dv=128, scale=0.088):
    return lib.zyfa_attn_fwd_bf16_paged(q, k, v, o, lse, cu, kvl, bt, n, maxs, maxp, nump, page, Hq, Hkv, T, Dqk, Dv,
                                        scale, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(o=MIS), INVALID), (dict(cu=None), INVALID),
    (dict(kvl=None), INVALID), (dict(bt=None), INVALID), (dict(kvl=0x90002), INVALID), (dict(bt=0xA0001), INVALID),
    (dict(n=0), INVALID), (dict(maxs=0), INVALID), (dict(maxs=1001), INVALID), (dict(maxp=0), INVALID),
    (dict(nump=0), INVALID), (dict(page=32), INVALID), (dict(page=192), INVALID), (dict(page=512), INVALID),
    (dict(maxp=1 << 23, page=256), INVALID), (dict(nump=1 << 30), INVALID), (dict(v=P2), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(scale=0.0), INVALID), (dict(Dqk=64, Dv=64), UNSUPPORTED),
    (dict(o=P), INVALID),
])
def test_paged_argument_checks(lib, kw, expect):
    assert bf16_paged(lib, **kw) == expect
    assert lib.zyfa_last_error() != b""
    assert fp8_paged(lib, **kw) == expect


@pytest.mark.parametrize("kw", [dict(qs=None), dict(ks=MIS), dict(blk=32), dict(lean=2), dict(page=64, blk=128)])
def test_fp8_paged_scale_and_mode_checks(lib, kw):
    assert fp8_paged(lib, **kw) == INVALID


WS = 0x1000000  # a 256-byte-aligned fake workspace


def fp8_decode(lib, q=P, k=P2, v=P3, qs=P4, ks=P5, vs=P6, blk=128, o=P7, lse=None, kvl=0x90000, bt=0xA0000, B=4,
               maxkv=1000, maxp=8, nump=30, page=128, Hq=8, Hkv=2, Dqk=128, Dv=128, scale=0.088, split=256, ws=WS,
               wsb=1 << 30, lean=0):
    return lib.zyfa_attn_decode_fp8_paged(q, k, v, qs, ks, vs, blk, o, lse, kvl, bt, B, maxkv, maxp, nump, page, Hq,
                                          Hkv, Dqk, Dv, scale, split, ws, wsb, lean, None)


def bf16_decode(lib, q=P, k=P2, v=P3, o=P7, lse=None, kvl=0x90000, bt=0xA0000, B=4, maxkv=1000, maxp=8, nump=30,
                page=128, Hq=8, Hkv=2, Dqk=128, Dv=128, scale=0.088, split=256, ws=WS, wsb=1 << 30):
    return lib.zyfa_attn_decode_bf16_paged(q, k, v, o, lse, kvl, bt, B, maxkv, maxp, nump, page, Hq, Hkv, Dqk, Dv,
                                           scale, split, ws, wsb, None)


def test_decode_workspace_bytes(lib):
    f = lib.zyfa_attn_decode_workspace_bytes
    assert f(4, 8, 128, 1000, 256) == (4 * 4 * 8 * 128 * 2 + 255) // 256 * 256 + 4 * 4 * 8 * 4
    assert f(4, 8, 128, 256, 256) == 0        # one split: results go straight to o / lse
    assert f(0, 8, 128, 1000, 256) == -1 and f(4, 8, 128, 1000, 0) == -1
    assert f(1 << 30, 1 << 30, 512, 1 << 30, 64) == -1  # would overflow
    assert f(1 << 30, 1 << 30, 126, 128, 64) == -1  # 2 parts of 2^60 rows: over the limit
    assert f(1 << 30, 1 << 30, 1 << 30, 1 << 30, 64) == -1
    # just under the limit: rows * (2 Dv + 4) * parts = 2^60 exactly
    rows, dv, parts = 1 << 40, 126, 1 << 12
    assert (2 * dv + 4) * rows * parts == 1 << 60
    assert f(1 << 20, 1 << 20, dv, parts * 64, 64) == (parts * rows * dv * 2 + 255) // 256 * 256 + parts * rows * 4
    assert f(1 << 20, (1 << 20) + 1, dv, parts * 64, 64) == -1


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(o=MIS), INVALID), (dict(kvl=None), INVALID), (dict(bt=0xA0002), INVALID),
    (dict(B=0), INVALID), (dict(maxkv=0), INVALID), (dict(maxkv=1025), INVALID), (dict(page=96), INVALID),
    (dict(split=0), INVALID), (dict(split=100), INVALID), (dict(ws=None), INVALID), (dict(ws=WS + 16), INVALID),
    (dict(wsb=1000), INVALID), (dict(ws=P7), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(Hq=512, Hkv=1), UNSUPPORTED), (dict(scale=-1.0), INVALID), (dict(Dqk=64, Dv=64), UNSUPPORTED),
    (dict(o=P), INVALID),
])
def test_decode_argument_checks(lib, kw, expect):
    assert bf16_decode(lib, **kw) == expect
    assert lib.zyfa_last_error() != b""
    assert fp8_decode(lib, **kw) == expect


def fp8_decode_noalloc(lib, q=P, k=P2, v=P3, qs=P4, ks=P5, vs=P6, blk=128, o=P7, lse=None, kvl=0x90000, bt=0xA0000, B=4,
                       maxkv=1000, maxp=8, nump=30, page=128, Hq=8, Hkv=2, Dqk=128, Dv=128, scale=0.088, split=256,
                       lean=0):
    return lib.zyfa_attn_decode_fp8_paged_noalloc(q, k, v, qs, ks, vs, blk, o, lse, kvl, bt, B, maxkv, maxp, nump, page,
                                                  Hq, Hkv, Dqk, Dv, scale, split, lean, None)


def test_decode_noalloc_checks():
    # the allocation-free decode rejects calls whose partial results exceed its 8 MiB scratch
    # array, before any device work, and otherwise checks its arguments as the decode with a
    # workspace does (these calls fail on the host: no GPU is touched)
    lib = _lib.load()
    big = dict(B=64, Hq=64, Hkv=8, maxkv=1 << 20, maxp=8192, split=64)
    need = lib.zyfa_attn_decode_workspace_bytes(64, 64, 128, 1 << 20, 64)
    assert need > 8 << 20
    assert fp8_decode_noalloc(lib, **big) == UNSUPPORTED
    assert b"8388608" in lib.zyfa_last_error()
    for kw in (dict(q=None), dict(o=MIS), dict(kvl=None), dict(B=0), dict(split=100), dict(lean=2), dict(blk=32),
               dict(scale=-1.0), dict(Dqk=64, Dv=64)):
        assert fp8_decode_noalloc(lib, **kw) in (INVALID, UNSUPPORTED), kw
        assert fp8_decode_noalloc(lib, **kw) == fp8_decode(lib, **kw), kw


@pytest.mark.parametrize("kw", [dict(qs=None), dict(vs=MIS), dict(blk=32), dict(lean=2), dict(page=64, blk=128)])
def test_fp8_decode_scale_and_mode_checks(lib, kw):
    assert fp8_decode(lib, **kw) == INVALID


def merge(lib, op=P, lp=P2, n=2, o=P3, lse=None, rows=1000, Dv=128):
    return lib.zyfa_attn_merge(op, lp, n, o, lse, rows, Dv, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(op=None), INVALID), (dict(lp=None), INVALID), (dict(o=None), INVALID), (dict(op=MIS), INVALID),
    (dict(lse=MIS), INVALID), (dict(n=0), INVALID), (dict(rows=0), INVALID), (dict(rows=-3), INVALID),
    (dict(Dv=100), UNSUPPORTED), (dict(Dv=192), UNSUPPORTED), (dict(o=P), INVALID), (dict(lse=P2), INVALID),
    (dict(lse=P3), INVALID), (dict(n=1 << 20, rows=1 << 20), INVALID),
])
def test_merge_argument_checks(lib, kw, expect):
    assert merge(lib, **kw) == expect
    assert lib.zyfa_last_error() != b""


def quant(lib, x=P, bf=0, codes=P2, scales=P3, B=1, H=2, S=100, D=128, blk=64, had=0):
    return lib.zyfa_quantize_fp8(x, bf, codes, scales, B, H, S, D, blk, had, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), INVALID), (dict(codes=None), INVALID), (dict(scales=None), INVALID), (dict(x=MIS), INVALID),
    (dict(bf=2), INVALID), (dict(had=3), INVALID), (dict(B=0), INVALID), (dict(S=0), INVALID), (dict(D=0), INVALID),
    (dict(blk=100), INVALID), (dict(D=64), UNSUPPORTED), (dict(D=64, had=1), UNSUPPORTED), (dict(codes=P), INVALID),
    (dict(D=192, had=2), INVALID),
])
def test_quantize_argument_checks(lib, kw, expect):
    assert quant(lib, **kw) == expect


BIG = (1 << 31) - 1


def test_size_checks_do_not_overflow(lib):
    # dimensions whose products pass 2^63: each is refused as too large, and no size check
    # forms such a product (the host sanitizer run of this file reports signed overflow)
    assert bf16(lib, B=BIG, Hq=BIG, Hkv=1, S=1 << 29) == INVALID
    assert fp8(lib, B=BIG, Hq=BIG, Hkv=1, S=1 << 29) == INVALID
    assert b"too large" in lib.zyfa_last_error()
    assert fp8_range(lib, B=BIG, Hq=BIG, Hkv=BIG, Sq=1 << 29, Skv=BIG, q_offset=0, k_end=1 << 20) == INVALID
    assert quant(lib, B=BIG, H=BIG, S=BIG, D=BIG) == INVALID
    assert b"too large" in lib.zyfa_last_error()
    assert merge(lib, n=8, rows=1 << 62) == INVALID
    assert b"too large" in lib.zyfa_last_error()
    # one sequence of 64 tokens, 2^24 heads (1 x 2^24 x 64 x 128 elements pass), a cache
    # of 2^31 - 1 pages of 256 tokens: 2^70 elements
    kw = dict(n=1, maxs=64, T=64, Hq=1 << 24, Hkv=1 << 24, maxp=1, nump=BIG, page=256)
    assert bf16_paged(lib, **kw) == INVALID
    assert fp8_paged(lib, **kw) == INVALID
    assert b"too large" in lib.zyfa_last_error()


def test_binding_takes_the_stream_of_one_device():
    import torch
    import fp8_causal_prefill_amd as z
    with pytest.raises(ValueError, match="one device"):
        z._stream(torch.zeros(1), torch.zeros(1, device="meta"))
    with pytest.raises(ValueError, match="one device"):
        z._stream(None, None)


def test_binding_raises_without_device_tensors():
    import torch
    import fp8_causal_prefill_amd as z
    with pytest.raises(ValueError):
        z.attn_fwd_bf16(torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16), torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16),
                        torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16))


def test_debug_env_reports_failures_on_stderr():
    # ZYFA_DEBUG=1: a rejected call also prints its status and message on stderr; without
    # it the library prints nothing (a child process, so that the variable is seen from the
    # start and stderr can be read)
    import subprocess
    import sys
    code = ("from fp8_causal_prefill_amd import _lib\n"
            "lib = _lib.load()\n"
            "st = lib.zyfa_attn_fwd_bf16(None, None, None, None, None, 1, 4, 2, 256, 128, 128, 0.088, None)\n"
            "assert st == 1, st\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=root)
    env.pop("ZYFA_DEBUG", None)
    quiet = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert quiet.returncode == 0, quiet.stderr
    assert "zyfa:" not in quiet.stderr
    env["ZYFA_DEBUG"] = "1"
    loud = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert loud.returncode == 0, loud.stderr
    assert "zyfa: ZYFA_ERR_INVALID_ARGUMENT: q, k, v and o must be non-null" in loud.stderr


def test_lds_poison_switch_reads_the_environment(monkeypatch):
    # the launchers' debug switch (ZYFA_LDS_POISON) follows the process environment at every
    # launch: unset or "0" is off, anything else on (the GPU side is tests/test_gpu_lds_poison.py)
    fn = ctypes.CDLL(_lib.LIB_PATH)._ZN4zyfa20lds_poison_requestedEv
    fn.restype = ctypes.c_bool
    monkeypatch.delenv("ZYFA_LDS_POISON", raising=False)
    assert not fn()
    monkeypatch.setenv("ZYFA_LDS_POISON", "1")
    assert fn()
    monkeypatch.setenv("ZYFA_LDS_POISON", "0")
    assert not fn()
    monkeypatch.setenv("ZYFA_LDS_POISON", "")
    assert not fn()


def test_timeline_build_exports_the_abi_and_its_readers():
    # libzyfa_timeline.so: the same entry points, plus the two readers of
    # include/zyfa_timeline.h; libzyfa.so has none of the latter
    from fp8_causal_prefill_amd.build import TIMELINE_LIB
    tl = ctypes.CDLL(TIMELINE_LIB)
    for n in declared_functions():
        assert hasattr(tl, n), n
    text = open(os.path.join(os.path.dirname(HEADER), "zyfa_timeline.h")).read()
    readers = sorted(set(re.findall(r"\b(zyfa_timeline_[a-z]+)\s*\(", text)))
    assert readers == ["zyfa_timeline_clear", "zyfa_timeline_read"]
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in readers:
        assert hasattr(tl, n) and not hasattr(raw, n), n
    tl.zyfa_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong]
    buf = (ctypes.c_ulonglong * 8)()
    assert tl.zyfa_timeline_read(None, 1) == 1  # hipErrorInvalidValue, before any HIP call
    assert tl.zyfa_timeline_read(buf, -1) == 1
    assert tl.zyfa_timeline_read(buf, 65537) == 1
