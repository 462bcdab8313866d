"""FP8 attention with block scales that are not powers of two and that vary from block to
block, through the C ABI, against the fp64 oracle on the same dequantized inputs.

The attention entry points accept any positive float32 scale per (batch, head, token
block). The quantizer only writes powers of two, so these tests take its codes and
multiply every Q, K and V block scale by a seeded factor in (1, 2); the inputs themselves
are scaled block by block (token block j by a power of two that cycles with j) so that
neighbouring blocks get different scales and a scale applied to the wrong block shows.
The oracle dequantizes with exactly the scales the kernel was given ("ZYFA", section
"Error of a Single Attention Call": fp64 attention on the same quantized inputs).

What is checked, for exact and lean probabilities ("Per-Block Scaling and Normalization by
the Rounded Row Sum": the V scale must not enter the probabilities or their row sum):

* O and the log-sum-exp against the oracle at D = 128 (GQA) and the MLA shape 192 / 128;
* the log-sum-exp does not depend on the V scales at all: bit for bit the same with
  power-of-two, non-power-of-two and subnormal V scales;
* split-KV windows merged by their log-sum-exps, a packed (varlen) batch, a paged cache
  (pages of 64 and 256 tokens) and decode with several key splits, each against its oracle.
"""

import math

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from oracle import (causal_attention, dequantize_blocks, paged_attention, varlen_attention,
                    window_attention)
from tests.paths import bf16_from_f64, rel_l2, to_dev
from workloads import custom, generate, page_table, scatter_pages

pytestmark = pytest.mark.gpu

BARS = {"fp8": 3e-2, "lean": 3e-2}
MODES = ["fp8", "lean"]


def _case(*a):
    print("case:", *a, flush=True)


def _lse_ok(mode, got, ref):
    # exact: a probability's e4m3 rounding moves the row sum by at most a factor 1 + 2^-4;
    # lean: a code in e4m3's normal range is off by at most 0.068 in log, and the weights
    # under 2^-13 of their block maximum add less than 2^-7 of it
    d = np.abs(got - ref)
    return d.max() < (math.log(1 + 2 ** -4) if mode == "fp8" else 0.1)


def _vary(x, block, period, low):
    """Scale token block j (token axis -2) by 2^((j mod period) + low)."""
    S = x.shape[-2]
    f = np.exp2(((np.arange(S) // block) % period) + low).astype(np.float32)
    return x * f[:, None]


def _mantissas(t, seed):
    """Block scales times seeded factors in (1, 2)."""
    rng = np.random.default_rng([4242, seed] + list(t.shape))
    m = torch.from_numpy(rng.uniform(1.0, 2.0, tuple(t.shape)).astype(np.float32)).to(t.device)
    return (t * m).contiguous()


def _quantize(x, block, seed):
    """GPU quantizer codes of x, with its block scales times factors in (1, 2)."""
    codes, scales = zy.quantize_fp8(to_dev(x), block)
    return codes, _mantissas(scales, seed)


def _deq(codes, scales, block):
    return dequantize_blocks(codes.cpu().numpy(), scales.cpu().numpy(), block)


def _inputs(B, Hq, Hkv, S, Dqk, Dv, block, seed, wid=930):
    q, k, v = generate(custom(B, Hq, Hkv, S, Dqk, Dv, wid=wid), seed=seed)
    return _vary(q, block, 3, -1), _vary(k, block, 3, -1), _vary(v, block, 5, 0)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(1, 4, 2, 700, 128, 64), (2, 2, 2, 600, 192, 128), (1, 2, 1, 1000, 128, 128)])
def test_non_power_of_two_scales_against_oracle(mode, shape):
    B, Hq, Hkv, S, Dqk, block = shape
    _case(mode, shape)
    q, k, v = _inputs(B, Hq, Hkv, S, Dqk, 128, block, seed=1)
    (qc, qs), (kc, ks), (vc, vs) = (_quantize(x, block, i) for i, x in enumerate((q, k, v)))
    tau = 1 / math.sqrt(Dqk)
    o, lse = zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, block, tau, return_lse=True, lean=mode == "lean")
    torch.cuda.synchronize()
    og, lg = bf16_from_f64(o), lse.cpu().numpy().astype(np.float64)
    ro, rl = causal_attention(_deq(qc, qs, block), _deq(kc, ks, block), _deq(vc, vs, block), tau)
    err = rel_l2(og, ro)
    print(f"{mode} rel-L2 {err:.3e}, max |dLSE| {np.abs(lg - rl).max():.3e}")
    assert err <= BARS[mode]
    assert _lse_ok(mode, lg, rl)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("Dqk", [128, 192])
def test_lse_does_not_depend_on_v_scales(mode, Dqk):
    B, Hq, Hkv, S, block = 1, 2, 1, 900, 128
    _case(mode, Dqk)
    q, k, v = _inputs(B, Hq, Hkv, S, Dqk, 128, block, seed=2)
    (qc, qs), (kc, ks) = _quantize(q, block, 0), _quantize(k, block, 1)
    vc, vs_pow2 = zy.quantize_fp8(to_dev(v), block)
    tau = 1 / math.sqrt(Dqk)
    # powers of two (the quantizer's), factors in (1, 2), and subnormal float32 scales
    # (2^-127 times factors in [0.5, 1): the V operand's E8M0 scale is then 2^-127)
    rng = np.random.default_rng(77)
    sub = torch.from_numpy((2.0 ** -127 * rng.uniform(0.5, 1.0, tuple(vs_pow2.shape))).astype(np.float32)).cuda()
    assert torch.all(sub < 2.0 ** -126) and torch.all(sub > 0)
    runs = {}
    for name, vs in (("pow2", vs_pow2), ("mantissa", _mantissas(vs_pow2, 2)), ("subnormal", sub)):
        o, lse = zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, block, tau, return_lse=True, lean=mode == "lean")
        torch.cuda.synchronize()
        runs[name] = (bf16_from_f64(o), lse.cpu().numpy(), vs)
    for name in ("mantissa", "subnormal"):
        assert np.array_equal(runs[name][1], runs["pow2"][1]), name
    qd, kd = _deq(qc, qs, block), _deq(kc, ks, block)
    for name, (og, lg, vs) in runs.items():
        ro, rl = causal_attention(qd, kd, _deq(vc, vs, block), tau)
        err = rel_l2(og, ro)
        print(f"{mode} {name} V scales: rel-L2 {err:.3e}")
        assert err <= BARS[mode]
        assert _lse_ok(mode, lg.astype(np.float64), rl)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("Dqk", [128, 192])
def test_non_power_of_two_scales_split_kv_and_merge(mode, Dqk):
    B, Hq, Hkv, S, block, edges = 1, 4, 2, 1000, 128, [0, 256, 640, 1000]
    _case(mode, Dqk, edges)
    q, k, v = _inputs(B, Hq, Hkv, S, Dqk, 128, block, seed=3)
    (qc, qs), (kc, ks), (vc, vs) = (_quantize(x, block, 10 + i) for i, x in enumerate((q, k, v)))
    deq = [_deq(qc, qs, block), _deq(kc, ks, block), _deq(vc, vs, block)]
    tau = 1 / math.sqrt(Dqk)
    o_parts, l_parts = [], []
    for lo, hi in zip(edges[:-1], edges[1:]):
        o, l = zy.attn_fwd_fp8_range(qc, kc, vc, qs, ks, vs, block, 0, lo, hi, tau, return_lse=True,
                                     lean=mode == "lean")
        torch.cuda.synchronize()
        on, ln = bf16_from_f64(o), l.cpu().numpy().astype(np.float64)
        ro, rl = window_attention(*deq, tau, k_begin=lo, k_end=hi)
        seen = np.isfinite(rl)
        assert np.array_equal(seen, np.isfinite(ln)) and np.all(on[~seen] == 0.0)
        assert rel_l2(on[seen], ro[seen]) <= BARS[mode]
        assert _lse_ok(mode, ln[seen], rl[seen])
        o_parts.append(o)
        l_parts.append(l)
    om, lm = zy.attn_merge(torch.stack(o_parts), torch.stack(l_parts), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = causal_attention(*deq, tau)
    err = rel_l2(bf16_from_f64(om), ro)
    print(f"{mode} merged rel-L2 {err:.3e}")
    assert err <= BARS[mode]
    assert _lse_ok(mode, lm.cpu().numpy().astype(np.float64), rl)


@pytest.mark.parametrize("mode", MODES)
def test_non_power_of_two_scales_varlen(mode):
    Hq, Hkv, D, block = 4, 2, 128, 64
    lengths = [300, 64, 1000, 129]
    _case(mode, lengths)
    cu = [0]
    for i, n in enumerate(lengths):
        cu.append(cu[-1] + (n if i == len(lengths) - 1 else -(-n // 64) * 64))
    cu = np.array(cu, dtype=np.int32)
    T = int(cu[-1]) + 21
    q, k, v = _inputs(1, Hq, Hkv, T, D, D, block, seed=4, wid=931)
    (qc, qs), (kc, ks), (vc, vs) = (_quantize(x, block, 20 + i) for i, x in enumerate((q, k, v)))
    o, lse = zy.attn_fwd_fp8_varlen(qc[0], kc[0], vc[0], qs[0], ks[0], vs[0], block, torch.from_numpy(cu).cuda(),
                                    int(np.max(np.diff(cu))), 1 / math.sqrt(D), return_lse=True,
                                    lean=mode == "lean")
    torch.cuda.synchronize()
    deq = [_deq(qc, qs, block)[0], _deq(kc, ks, block)[0], _deq(vc, vs, block)[0]]
    ro, rl = varlen_attention(*deq, 1 / math.sqrt(D), cu)
    inside = np.isfinite(rl[0])
    og, lg = bf16_from_f64(o), lse.cpu().numpy().astype(np.float64)
    err = rel_l2(og[:, inside], ro[:, inside])
    print(f"{mode} varlen rel-L2 {err:.3e}")
    assert err <= BARS[mode]
    assert _lse_ok(mode, lg[:, inside], rl[:, inside])


class _Cache:
    """Sequences of kv_lens tokens scattered into a shuffled page cache; each page's token
    blocks scaled by a power of two that cycles with the page index and the block."""

    def __init__(self, kv_lens, P, Hkv, Dqk, Dv, block, seed):
        self.kv_lens = np.array(kv_lens, dtype=np.int32)
        self.table, self.num_pages = page_table(kv_lens, P, seed)
        rng = np.random.default_rng([932, seed])
        self.k = rng.standard_normal((self.num_pages, Hkv, P, Dqk), dtype=np.float32)
        self.v = rng.standard_normal((self.num_pages, Hkv, P, Dv), dtype=np.float32)
        for i, n in enumerate(kv_lens):
            _, k, v = generate(custom(1, Hkv, Hkv, n, Dqk, Dv, wid=933 + i), seed=seed)
            scatter_pages(self.k, self.table[i], k[0])
            scatter_pages(self.v, self.table[i], v[0])
        pg = np.arange(self.num_pages)[:, None, None, None]
        blk = (np.arange(P) // block)[None, None, :, None]
        self.k *= np.exp2(((pg + blk) % 3) - 1).astype(np.float32)
        self.v *= np.exp2((3 * pg + blk) % 5).astype(np.float32)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("P", [64, 256])
def test_non_power_of_two_scales_paged(mode, P):
    Hq, Hkv, D = 4, 2, 128
    block = 64
    seqs = [(700, 300), (1500, 37), (300, 300)]
    _case(mode, P, seqs)
    kv, ch = zip(*seqs)
    pad = [0 if i == len(ch) - 1 else -(-n // 64) * 64 - n for i, n in enumerate(ch)]
    kv = [n + p for n, p in zip(kv, pad)]
    cu = np.cumsum([0] + [n + p for n, p in zip(ch, pad)]).astype(np.int32)
    T = int(cu[-1])
    c = _Cache(kv, P, Hkv, D, D, block, seed=5)
    q, _, _ = generate(custom(1, Hq, Hq, T, D, D, wid=940), seed=5)
    qc, qs = _quantize(_vary(q, block, 3, -1), block, 30)
    kc, ks = _quantize(c.k, block, 31)
    vc, vs = _quantize(c.v, block, 32)
    o, lse = zy.attn_fwd_fp8_paged(qc[0], kc, vc, qs[0], ks, vs, block, torch.from_numpy(cu).cuda(),
                                   torch.from_numpy(c.kv_lens).cuda(), torch.from_numpy(c.table).cuda(),
                                   int(np.max(np.diff(cu))), 1 / math.sqrt(D), return_lse=True, lean=mode == "lean")
    torch.cuda.synchronize()
    ro, rl = paged_attention(_deq(qc, qs, block)[0], _deq(kc, ks, block), _deq(vc, vs, block), 1 / math.sqrt(D), cu,
                             c.kv_lens, c.table)
    og, lg = bf16_from_f64(o), lse.cpu().numpy().astype(np.float64)
    err = rel_l2(og, ro)
    print(f"{mode} paged rel-L2 {err:.3e}")
    assert err <= BARS[mode]
    assert _lse_ok(mode, lg, rl)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(8, 2, 128), (4, 4, 192)])
def test_non_power_of_two_scales_decode(mode, shape):
    Hq, Hkv, Dqk = shape
    Dv, P, block = 128, 128, 64
    kv_lens = [1, 65, 700, 1500, 2048]
    B = len(kv_lens)
    _case(mode, shape, kv_lens)
    c = _Cache(kv_lens, P, Hkv, Dqk, Dv, block, seed=6)
    q, _, _ = generate(custom(1, B, B, Hq, Dqk, Dv, wid=941), seed=6)
    g = Hq // Hkv
    qc, qs = _quantize(q[0].reshape(B, Hkv, g, Dqk), block, 40)  # one scale per KV group
    kc, ks = _quantize(c.k, block, 41)
    vc, vs = _quantize(c.v, block, 42)
    kvl, bt = torch.from_numpy(c.kv_lens).cuda(), torch.from_numpy(c.table).cuda()
    qd = _deq(qc, qs, block).reshape(B, Hq, Dqk)
    ref = paged_attention(np.ascontiguousarray(qd.transpose(1, 0, 2)), _deq(kc, ks, block), _deq(vc, vs, block),
                          1 / math.sqrt(Dqk), np.arange(B + 1), c.kv_lens, c.table)
    ro, rl = ref[0].transpose(1, 0, 2), ref[1].T
    for split in (128, 512):  # 16 and 4 key splits of the longest sequence, merged by their LSE
        o, lse = zy.attn_decode_fp8_paged(qc.reshape(B, Hq, Dqk), kc, vc, qs, ks, vs, block, kvl, bt, max(kv_lens),
                                          split_keys=split, return_lse=True, lean=mode == "lean")
        torch.cuda.synchronize()
        og, lg = bf16_from_f64(o), lse.cpu().numpy().astype(np.float64)
        err = rel_l2(og, ro)
        print(f"{mode} decode split {split} rel-L2 {err:.3e}")
        assert err <= BARS[mode]
        assert _lse_ok(mode, lg, rl)
