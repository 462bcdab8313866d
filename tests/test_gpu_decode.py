"""GPU decode (one new token per sequence) against a paged key/value cache, through the C
ABI, against the fp64 oracle on the same inputs.

The oracle is paged_attention with a chunk of one token per sequence (row at position
kv_len - 1, seeing every key). Bars as for the whole-sequence calls over all outputs:
BF16 <= 5e-3, FP8 (exact and lean) <= 3e-2 (the splits' partial outputs are rounded to
bfloat16 before the merge, which adds at most about one bfloat16 rounding). Beyond the
bars: with one split and BF16 inputs, decode equals the paged prefill call with a
one-token chunk per sequence, bit for bit (both take the same tiles in the same order for
the row); results do not depend on the split beyond the partials' rounding; a malformed
kv_lens entry gives O = 0 and LSE = -inf for its sequence only.
"""

import math

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from oracle import dequantize_blocks, paged_attention
from tests.paths import bf16_from_f64, rel_l2, to_dev
from workloads import custom, generate, page_table, scatter_pages

pytestmark = pytest.mark.gpu

BARS = {"fp8": 3e-2, "lean": 3e-2, "bf16": 5e-3}


def _case(*a):
    print("case:", *a, flush=True)


class Decode:
    """B sequences of kv_lens tokens in a shuffled page cache, and one query per sequence
    and query head."""

    def __init__(self, kv_lens, P, Hq, Hkv, Dqk, Dv, seed):
        self.kv_lens = np.array(kv_lens, dtype=np.int32)
        self.B, self.Hq, self.Hkv, self.P = len(kv_lens), Hq, Hkv, P
        self.table, self.num_pages = page_table(kv_lens, P, seed)
        rng = np.random.default_rng([905, seed])
        self.k = rng.standard_normal((self.num_pages, Hkv, P, Dqk), dtype=np.float32)
        self.v = rng.standard_normal((self.num_pages, Hkv, P, Dv), dtype=np.float32)
        q, _, _ = generate(custom(1, self.B, self.B, Hq, Dqk, Dv, wid=906), seed=seed)
        self.q = q[0]                                     # [B, Hq, Dqk]
        for i, n in enumerate(kv_lens):
            _, k, v = generate(custom(1, Hkv, Hkv, n, Dqk, Dv, wid=907 + i), seed=seed)
            scatter_pages(self.k, self.table[i], k[0])
            scatter_pages(self.v, self.table[i], v[0])

    def run(self, mode, block=64, split_keys=None, kv_lens=None, max_kv_len=None):
        kvl = torch.from_numpy(self.kv_lens if kv_lens is None else np.array(kv_lens, dtype=np.int32)).cuda()
        bt = torch.from_numpy(self.table).cuda()
        mkv = int(self.kv_lens.max()) if max_kv_len is None else max_kv_len
        g = self.Hq // self.Hkv
        if mode == "bf16":
            t = [to_dev(x).to(torch.bfloat16) for x in (self.q, self.k, self.v)]
            o, lse = zy.attn_decode_bf16_paged(*t, kvl, bt, mkv, split_keys=split_keys, return_lse=True)
            deq = [x.float().cpu().numpy().astype(np.float64) for x in t]
        else:
            B, Hq, D = self.q.shape
            qc, qs = zy.quantize_fp8(to_dev(self.q).reshape(B, self.Hkv, g, D), block)  # one scale per KV group
            kc, ks = zy.quantize_fp8(to_dev(self.k), block)
            vc, vs = zy.quantize_fp8(to_dev(self.v), block)
            o, lse = zy.attn_decode_fp8_paged(qc.reshape(B, Hq, D), kc, vc, qs, ks, vs, block, kvl, bt, mkv,
                                              split_keys=split_keys, return_lse=True, lean=mode == "lean")
            deq = [dequantize_blocks(qc.cpu().numpy(), qs.cpu().numpy(), block).reshape(B, Hq, D),
                   dequantize_blocks(kc.cpu().numpy(), ks.cpu().numpy(), block),
                   dequantize_blocks(vc.cpu().numpy(), vs.cpu().numpy(), block)]
        torch.cuda.synchronize()
        return bf16_from_f64(o), lse.cpu().numpy().astype(np.float64), deq

    def oracle(self, deq, scale, kv_lens=None):
        kvl = self.kv_lens if kv_lens is None else np.array(kv_lens)
        q = np.ascontiguousarray(deq[0].transpose(1, 0, 2))       # [Hq, B, D]: one-token chunks
        o, lse = paged_attention(q, deq[1], deq[2], scale, np.arange(self.B + 1), kvl, self.table)
        return o.transpose(1, 0, 2), lse.T


KV = [1, 63, 64, 65, 700, 1500, 129, 2048]


@pytest.mark.parametrize("mode", ["bf16", "fp8", "lean"])
@pytest.mark.parametrize("P", [64, 256])
@pytest.mark.parametrize("shape", [(8, 2, 128, 128), (32, 1, 128, 128), (4, 4, 192, 128)])
@pytest.mark.parametrize("split_keys", [128, None, 4096])
def test_decode_against_oracle(mode, P, shape, split_keys):
    Hq, Hkv, Dqk, Dv = shape
    _case(mode, P, shape, split_keys)
    d = Decode(KV, P, Hq, Hkv, Dqk, Dv, seed=1)
    og, lg, deq = d.run(mode, block=64 if P == 64 else 128, split_keys=split_keys)
    ro, rl = d.oracle(deq, 1 / math.sqrt(Dqk))
    err = rel_l2(og, ro)
    print(f"{mode} decode rel-L2 {err:.3e}")
    assert err <= BARS[mode]
    dl = np.abs(lg - rl)
    assert dl.max() < (1e-3 if mode == "bf16" else (math.log(1 + 2 ** -4) if mode == "fp8" else 0.1))
    # the first sequence has one key: its output is that key's value
    assert rel_l2(og[0], np.repeat(deq[2][d.table[0, 0], :, 0][:, None], Hq // Hkv, axis=1).reshape(Hq, Dv)) < 8e-3


def test_decode_bf16_one_split_is_the_paged_prefill_call():
    Hq, Hkv, D, P = 8, 2, 128, 128
    _case("bf16 decode = paged prefill")
    d = Decode(KV, P, Hq, Hkv, D, D, seed=2)
    kvl = torch.from_numpy(d.kv_lens).cuda()
    bt = torch.from_numpy(d.table).cuda()
    q, k, v = (to_dev(x).to(torch.bfloat16) for x in (d.q, d.k, d.v))
    o1, l1 = zy.attn_decode_bf16_paged(q, k, v, kvl, bt, int(d.kv_lens.max()), split_keys=4096, return_lse=True)
    # each sequence's token as a one-token chunk of the paged prefill call
    for i in range(d.B):
        cu = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
        o2, l2 = zy.attn_fwd_bf16_paged(q[i][:, None].contiguous(), k, v, cu, kvl[i:i + 1].contiguous(),
                                        bt[i:i + 1].contiguous(), 1, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o1[i], o2[:, 0]) and torch.equal(l1[i], l2[:, 0]), i


@pytest.mark.parametrize("mode", ["bf16", "fp8"])
def test_decode_split_invariance_and_malformed(mode):
    Hq, Hkv, D, P = 8, 2, 128, 128
    _case(mode, "splits / malformed")
    d = Decode(KV, P, Hq, Hkv, D, D, seed=3)
    o1, l1, _ = d.run(mode, split_keys=4096)
    for sk in (64, 192, 1024):
        o2, l2, _ = d.run(mode, split_keys=sk)
        assert rel_l2(o2, o1) < 4e-3 and np.max(np.abs(l2 - l1)) < 1e-4
    bad = [int(n) for n in d.kv_lens]
    bad[2] = 0            # no token
    bad[4] = 5000         # beyond max_kv_len
    o3, l3, deq = d.run(mode, split_keys=256, kv_lens=bad, max_kv_len=int(d.kv_lens.max()))
    assert np.all(o3[[2, 4]] == 0.0) and np.all(l3[[2, 4]] == -np.inf)
    keep = [i for i in range(d.B) if i not in (2, 4)]
    assert rel_l2(o3[keep], o1[keep]) < 4e-3


@pytest.mark.parametrize("mode", ["bf16", "fp8"])
def test_decode_large_group_on_the_eight_wave_workgroup(mode):
    # 64 query heads per KV head: more rows than one wave holds, so the eight-wave
    # workgroup runs; six of its waves lie past the rows (BF16: they take only their share
    # of the copies; FP8: they compute clamped rows that are not stored)
    Hq, Hkv, D, P = 64, 1, 128, 128
    _case(mode, "64 heads per KV head")
    d = Decode([1, 65, 700, 2048], P, Hq, Hkv, D, D, seed=4)
    for sk in (128, 4096):
        og, lg, deq = d.run(mode, block=64, split_keys=sk)
        ro, rl = d.oracle(deq, 1 / math.sqrt(D))
        err = rel_l2(og, ro)
        print(f"{mode} split {sk} rel-L2 {err:.3e}")
        assert err <= BARS[mode]
        assert np.abs(lg - rl).max() < (1e-3 if mode == "bf16" else math.log(1 + 2 ** -4))
