"""Tensors past 2^31 elements: 64 batch entries of 64 query heads (8 key/value heads),
4096 tokens, D = 128, so that Q and O hold 2^31 elements and the last head's rows sit past
every 32-bit element offset.

Inputs are drawn on the device from a seeded generator (e4m3 codes without NaN codes and
power-of-two block scales for FP8, bfloat16 normals for BF16). Checked, for the first and
the last (batch, query head): the rows equal, bit for bit, those of a call on that head's
slices alone (B = Hq = Hkv = 1), and sampled rows match the fp64 oracle on the very codes
(or bfloat16 values) the kernel read, within the FP8 and BF16 bars.
"""

import math

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from oracle import causal_attention, dequantize_blocks

pytestmark = pytest.mark.gpu

B, HQ, HKV, S, D, BLOCK = 64, 64, 8, 4096, 128, 128
ROWS = np.array([0, 1, 777, 2048, S - 1])
HEADS = [(0, 0), (B - 1, HQ - 1)]


def _case(*a):
    print("case:", *a, flush=True)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _oracle_rows(q, k, v, rows):
    """fp64 causal attention of the given rows of one head (q [S, D], k, v [S, D] float64)."""
    o, lse = causal_attention(q[None, None], k[None, None], v[None, None], 1.0 / math.sqrt(D), rows=rows)
    return o[0, 0], lse[0, 0]


def test_fp8_past_2_31_elements():
    _case("fp8", B, HQ, HKV, S, D)
    assert B * HQ * S * D == 2 ** 31
    g = torch.Generator(device="cuda").manual_seed(31)

    def codes(h):  # |value| < 1 (codes below 0x40) with a random sign: no NaN code
        c = torch.randint(0, 0x40, (B, h, S, D), generator=g, device="cuda", dtype=torch.uint8)
        return c | (torch.randint(0, 2, (B, h, S, D), generator=g, device="cuda", dtype=torch.uint8) << 7)

    def scales(h):
        return torch.exp2(torch.randint(-2, 2, (B, h, S // BLOCK), generator=g, device="cuda").float())

    q, k, v = codes(HQ), codes(HKV), codes(HKV)
    qs, ks, vs = scales(HQ), scales(HKV), scales(HKV)
    o, lse = zy.attn_fwd_fp8(q, k, v, qs, ks, vs, BLOCK, return_lse=True)
    torch.cuda.synchronize()
    for b, h in HEADS:
        hk = h // (HQ // HKV)
        sl = lambda t, hh: t[b:b + 1, hh:hh + 1].contiguous()
        o1, l1 = zy.attn_fwd_fp8(sl(q, h), sl(k, hk), sl(v, hk), sl(qs, h), sl(ks, hk), sl(vs, hk), BLOCK,
                                 return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o[b, h], o1[0, 0]) and torch.equal(lse[b, h], l1[0, 0]), (b, h)
        deq = [dequantize_blocks(sl(t, hh).cpu().numpy(), sl(s, hh).cpu().numpy(), BLOCK)[0, 0]
               for t, s, hh in ((q, qs, h), (k, ks, hk), (v, vs, hk))]
        ro, rl = _oracle_rows(*deq, ROWS)
        got = o[b, h, ROWS].float().cpu().numpy().astype(np.float64)
        err = _rel(got, ro)
        print(f"fp8 (b={b}, h={h}) sampled rows rel-L2 {err:.3e}", flush=True)
        assert err <= 3e-2
        assert np.max(np.abs(lse[b, h, ROWS].cpu().numpy() - rl)) < math.log(1 + 2 ** -4)
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_bf16_past_2_31_elements():
    _case("bf16", B, HQ, HKV, S, D)
    g = torch.Generator(device="cuda").manual_seed(32)
    q = torch.randn((B, HQ, S, D), generator=g, device="cuda", dtype=torch.bfloat16)
    k = torch.randn((B, HKV, S, D), generator=g, device="cuda", dtype=torch.bfloat16)
    v = torch.randn((B, HKV, S, D), generator=g, device="cuda", dtype=torch.bfloat16)
    o, lse = zy.attn_fwd_bf16(q, k, v, return_lse=True)
    torch.cuda.synchronize()
    for b, h in HEADS:
        hk = h // (HQ // HKV)
        sl = lambda t, hh: t[b:b + 1, hh:hh + 1].contiguous()
        o1, l1 = zy.attn_fwd_bf16(sl(q, h), sl(k, hk), sl(v, hk), return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o[b, h], o1[0, 0]) and torch.equal(lse[b, h], l1[0, 0]), (b, h)
        deq = [t[b, hh].float().cpu().numpy().astype(np.float64) for t, hh in ((q, h), (k, hk), (v, hk))]
        ro, rl = _oracle_rows(*deq, ROWS)
        got = o[b, h, ROWS].float().cpu().numpy().astype(np.float64)
        err = _rel(got, ro)
        print(f"bf16 (b={b}, h={h}) sampled rows rel-L2 {err:.3e}", flush=True)
        assert err <= 5e-3
        assert np.max(np.abs(lse[b, h, ROWS].cpu().numpy() - rl)) < 1e-3
    del q, k, v, o, lse
    torch.cuda.empty_cache()
