"""Performance regression thresholds on the GPU: the headline kernels, decode and a short
sequence, timed with HIP events over rounds of back-to-back calls (the median round's
mean, after 3 unrecorded calls), each against a ceiling about 30 % above its usual time.

Boxes of the same model differ by up to about 7 % here (clocks under the board's power
limit differ), so the ceilings are loose: they catch a change that costs a kernel a
fifth or more (a lost overlap, a spill in the loop, a serialised copy), not noise. Usual
times on this board: FP8 exact 4.3-4.7 ms, lean 4.2-4.6 ms, BF16 7.0-7.6 ms at the
headline shape; decode of 8 x 32K keys 0.10 ms; FP8 at 4K tokens, 32 heads 0.083-0.088 ms
(0.09 ms through the Python binding, whose host work per call shows at this size).
Inputs are standard normal (as the benchmark's), drawn on the device from a fixed seed."""

import math

import pytest
import torch

import fp8_causal_prefill_amd as zy

pytestmark = pytest.mark.gpu


def _median_ms(fn, calls=10, rounds=5, warmup=3):
    """Median over rounds of the mean time of `calls` back-to-back calls (launch gaps
    amortised as in the benchmark)."""
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    per_call = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            fn()
        e1.record(stream)
        e1.synchronize()
        per_call.append(e0.elapsed_time(e1) / calls)
    per_call.sort()
    return per_call[len(per_call) // 2]


def _operands(B, Hq, Hkv, S, D, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((B, Hq, S, D), generator=g, device="cuda")
    k = torch.randn((B, Hkv, S, D), generator=g, device="cuda")
    v = torch.randn((B, Hkv, S, D), generator=g, device="cuda")
    return q, k, v


def _check(name, ms, ceiling):
    print(f"{name}: {ms:.4f} ms (ceiling {ceiling} ms)", flush=True)
    assert ms <= ceiling, f"{name} took {ms:.4f} ms, over its regression ceiling of {ceiling} ms"


def test_headline_kernels_within_their_ceilings():
    B, Hq, Hkv, S, D = 1, 32, 8, 32768, 128
    q, k, v = _operands(B, Hq, Hkv, S, D, seed=11)
    qc, qs = zy.quantize_fp8(q, 128)
    kc, ks = zy.quantize_fp8(k, 128)
    vc, vs = zy.quantize_fp8(v, 128)
    qb, kb, vb = q.bfloat16(), k.bfloat16(), v.bfloat16()
    del q, k, v
    o = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device="cuda")
    tau = 1 / math.sqrt(D)
    _check("FP8 exact, 32K", _median_ms(lambda: zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, 128, tau, o=o)), 5.8)
    _check("FP8 lean, 32K", _median_ms(lambda: zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, 128, tau, o=o, lean=True)), 5.7)
    _check("BF16, 32K", _median_ms(lambda: zy.attn_fwd_bf16(qb, kb, vb, tau, o=o)), 9.6)


def test_short_sequence_within_its_ceiling():
    B, Hq, Hkv, S, D = 1, 32, 32, 4096, 128
    q, k, v = _operands(B, Hq, Hkv, S, D, seed=12)
    qc, qs = zy.quantize_fp8(q, 128)
    kc, ks = zy.quantize_fp8(k, 128)
    vc, vs = zy.quantize_fp8(v, 128)
    o = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device="cuda")
    _check("FP8 exact, 4K", _median_ms(lambda: zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, 128, o=o), calls=30), 0.115)


def test_decode_within_its_ceiling():
    # 8 sequences of 32768 keys, 32 query and 8 KV heads, D = 128, 128-token pages in a
    # shuffled cache, FP8 exact with the default key splits
    B, Hq, Hkv, L, D, P = 8, 32, 8, 32768, 128, 128
    pages_per_seq = L // P
    num_pages = B * pages_per_seq
    g = torch.Generator(device="cuda").manual_seed(13)
    kc, ks = zy.quantize_fp8(torch.randn((num_pages, Hkv, P, D), generator=g, device="cuda"), 128)
    vc, vs = zy.quantize_fp8(torch.randn((num_pages, Hkv, P, D), generator=g, device="cuda"), 128)
    table = torch.randperm(num_pages, generator=g, device="cuda").to(torch.int32).reshape(B, pages_per_seq)
    kv_lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = torch.randn((B, Hkv, Hq // Hkv, D), generator=g, device="cuda")
    qc, qs = zy.quantize_fp8(q, 128)
    qc = qc.reshape(B, Hq, D)
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    _check("FP8 decode, 8 x 32K", _median_ms(
        lambda: zy.attn_decode_fp8_paged(qc, kc, vc, qs, ks, vs, 128, kv_lens, table, L, o=o), calls=30), 0.14)
