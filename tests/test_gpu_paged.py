"""GPU prefill against a paged key/value cache, through the C ABI, against the fp64 oracle
on the same inputs.

Each sequence's keys and values sit in pages of a shared cache, in a seeded random page
order; its chunk of new tokens is the last L of its kv_len tokens. Bars as for the
whole-sequence calls (relative L2 over the rows of all chunks: BF16 <= 5e-3, FP8 <= 3e-2,
lean the same). Beyond the bars: every chunk equals the range call (q_offset = kv_len - L) on
its pages gathered into one contiguous sequence, bit for bit (same codes and scales); rows
outside every chunk keep what the output held; a sequence whose entries break the rules
is left unwritten while the others are computed, and a page index outside the cache is
clamped into it (no read leaves the cache).
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
SENTINEL = 7.0


def _case(*a):
    print("case:", *a, flush=True)


class Paged:
    """One batch: chunks packed along the token axis (starts on multiples of 64), each
    sequence's keys and values scattered into a shuffled page cache (the rest of the
    cache holds unrelated random values)."""

    def __init__(self, kv_lens, chunk_lens, P, Hq, Hkv, Dqk, Dv, seed, tail=13):
        # each chunk but the last padded at its end to a multiple of 64 rows; the padding
        # tokens follow the sequence's own in the cache too (counted in its kv_len)
        pad = [0 if i == len(chunk_lens) - 1 else -(-n // 64) * 64 - n for i, n in enumerate(chunk_lens)]
        kv_lens = [n + p for n, p in zip(kv_lens, pad)]
        self.kv_lens = np.array(kv_lens, dtype=np.int32)
        self.P = P
        cu = [0]
        for n, p in zip(chunk_lens, pad):
            cu.append(cu[-1] + n + p)
        self.cu = np.array(cu, dtype=np.int32)
        self.T = int(cu[-1]) + tail
        self.table, self.num_pages = page_table(kv_lens, P, seed)
        self.max_seqlen = max(1, int(np.max(np.diff(self.cu))))
        rng = np.random.default_rng([901, seed])
        self.k = rng.standard_normal((self.num_pages, Hkv, P, Dqk), dtype=np.float32)
        self.v = rng.standard_normal((self.num_pages, Hkv, P, Dv), dtype=np.float32)
        q, _, _ = generate(custom(1, Hq, Hq, self.T, Dqk, Dv, wid=902), seed=seed)
        self.q = q[0]
        for i, n in enumerate(kv_lens):
            _, k, v = generate(custom(1, Hkv, Hkv, n, Dqk, Dv, wid=903 + i), seed=seed)
            scatter_pages(self.k, self.table[i], k[0])
            scatter_pages(self.v, self.table[i], v[0])

    def dev_meta(self):
        return (torch.from_numpy(self.cu).cuda(), torch.from_numpy(self.kv_lens).cuda(),
                torch.from_numpy(self.table).cuda())

    def run(self, mode, block=64, table=None, kv_lens=None):
        """GPU call; returns (o, lse) device tensors and the dequantized values the kernel
        reads (q, k_cache, v_cache float64) and the device operands."""
        Hq, T = self.q.shape[:2]
        o = torch.full((Hq, T, self.v.shape[3]), SENTINEL, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((Hq, T), SENTINEL, dtype=torch.float32, device="cuda")
        cu, kvl, bt = self.dev_meta()
        if table is not None:
            bt = torch.from_numpy(table).cuda()
        if kv_lens is not None:
            kvl = torch.from_numpy(np.array(kv_lens, dtype=np.int32)).cuda()
        if mode == "bf16":
            t = [to_dev(x).to(torch.bfloat16) for x in (self.q, self.k, self.v)]
            zy.attn_fwd_bf16_paged(*t, cu, kvl, bt, self.max_seqlen, o=o, lse=lse)
            deq = [x.float().cpu().numpy().astype(np.float64) for x in t]
            ops = (t, None)
        else:
            qc, qs = zy.quantize_fp8(to_dev(self.q)[None], block)
            kc, ks = zy.quantize_fp8(to_dev(self.k), block)   # the cache as [pages, Hkv, P, D]
            vc, vs = zy.quantize_fp8(to_dev(self.v), block)
            zy.attn_fwd_fp8_paged(qc[0], kc, vc, qs[0], ks, vs, block, cu, kvl, bt, self.max_seqlen, o=o, lse=lse,
                                  lean=mode == "lean")
            deq = [dequantize_blocks(qc.cpu().numpy(), qs.cpu().numpy(), block)[0],
                   dequantize_blocks(kc.cpu().numpy(), ks.cpu().numpy(), block),
                   dequantize_blocks(vc.cpu().numpy(), vs.cpu().numpy(), block)]
            ops = ((qc[0], kc, vc), (qs[0], ks, vs))
        torch.cuda.synchronize()
        return o, lse, deq, ops

    def inside(self):
        m = np.zeros(self.T, dtype=bool)
        for s0, s1 in zip(self.cu[:-1], self.cu[1:]):
            m[s0:s1] = True
        return m


# (kv_len, chunk length): a chunk at the end of a long prefix, a whole sequence of one
# page, a short chunk, a whole sequence, an empty chunk, a one-token chunk
SEQS = [(700, 300), (64, 64), (1500, 37), (300, 300), (129, 0), (1000, 1)]


@pytest.mark.parametrize("mode", ["bf16", "fp8", "lean"])
@pytest.mark.parametrize("P", [64, 128, 256])
@pytest.mark.parametrize("shape", [(4, 2, 128, 128), (2, 2, 192, 128)])
def test_paged_against_oracle(mode, P, shape):
    Hq, Hkv, Dqk, Dv = shape
    _case(mode, P, shape)
    kv, ch = zip(*SEQS)
    b = Paged(kv, ch, P, Hq, Hkv, Dqk, Dv, seed=1)
    o, lse, deq, _ = b.run(mode, block=64 if P == 64 else 128)
    ro, rl = paged_attention(deq[0], deq[1], deq[2], 1 / math.sqrt(Dqk), b.cu, b.kv_lens, b.table)
    inside = b.inside()
    og, lg = bf16_from_f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.all(og[:, ~inside] == SENTINEL) and np.all(lg[:, ~inside] == SENTINEL)
    err = rel_l2(og[:, inside], ro[:, inside])
    print(f"{mode} paged rel-L2 {err:.3e}")
    assert err <= BARS[mode]
    d = np.abs(lg[:, inside] - rl[:, inside])
    assert d.max() < (1e-3 if mode == "bf16" else (math.log(1 + 2 ** -4) if mode == "fp8" else 0.1))


def _gather(x, table_row, n):
    """[pages, H, P, ...] device tensor -> the sequence's first n positions [H, n, ...]."""
    P = x.shape[2]
    pages = torch.from_numpy(table_row[:-(-n // P)].astype(np.int64)).cuda()
    g = x[pages].transpose(0, 1)                     # [H, n_pages, P, ...]
    return g.reshape(g.shape[0], -1, *g.shape[3:])[:, :n].contiguous()


@pytest.mark.parametrize("mode", ["bf16", "fp8", "lean"])
@pytest.mark.parametrize("P", [64, 256])
def test_paged_is_the_range_call_on_gathered_pages(mode, P):
    Hq, Hkv, D = 4, 1, 128
    _case(mode, P, "gathered")
    kv, ch = zip(*SEQS)
    b = Paged(kv, ch, P, Hq, Hkv, D, D, seed=2)
    blk = 64
    o, lse, _, (t, s) = b.run(mode, block=blk)
    for i, (s0, s1) in enumerate(zip(b.cu[:-1], b.cu[1:])):
        n, L = int(b.kv_lens[i]), int(s1 - s0)
        if L == 0:
            continue
        q = t[0][:, s0:s1].clone()[None]
        k, v = (_gather(x, b.table[i], n)[None] for x in t[1:])
        if mode == "bf16":
            op, lp = zy.attn_fwd_bf16_range(q, k, v, n - L, return_lse=True)
        else:
            qs = s[0][:, s0 // blk:-(-s1 // blk)].clone()[None]
            ks, vs = (_gather(x[:, :, :, None], b.table[i], -(-n // blk))[..., 0][None] for x in s[1:])
            op, lp = zy.attn_fwd_fp8_range(q, k, v, qs, ks, vs, blk, n - L, return_lse=True, lean=mode == "lean")
        torch.cuda.synchronize()
        assert torch.equal(op[0], o[:, s0:s1]) and torch.equal(lp[0], lse[:, s0:s1]), (i, n, L)


@pytest.mark.parametrize("mode", ["bf16", "fp8"])
def test_paged_malformed_entries(mode):
    Hq, Hkv, D, P = 2, 2, 128, 128
    _case(mode, "malformed")
    seqs = [(500, 200), (400, 300), (900, 150), (256, 100)]
    kv, ch = zip(*seqs)
    b = Paged(kv, ch, P, Hq, Hkv, D, D, seed=3)
    table = b.table.copy()
    table[2, 1] = b.num_pages + 5      # outside the cache: clamped to its last page
    table[2, 3] = -7                   # clamped to page 0
    kv_bad = [int(n) for n in b.kv_lens]   # (with the chunks' padding)
    kv_bad[1] = 250                    # fewer tokens than the chunk: left unwritten
    kv_bad[3] = 10 ** 6                # more than the table holds: left unwritten
    o, lse, deq, _ = b.run(mode, block=128, table=table, kv_lens=kv_bad)
    og, lg = bf16_from_f64(o), lse.cpu().numpy()
    for i in (1, 3):
        s0, s1 = b.cu[i], b.cu[i + 1]
        assert np.all(og[:, s0:s1] == SENTINEL) and np.all(lg[:, s0:s1] == SENTINEL)
    # sequence 2 reads the pages its clamped entries name: the oracle on that table
    clamped = np.clip(table, 0, b.num_pages - 1)
    ro, _ = paged_attention(deq[0], deq[1], deq[2], 1 / math.sqrt(D), b.cu, b.kv_lens, clamped)
    for i in (0, 2):
        s0, s1 = b.cu[i], b.cu[i + 1]
        assert rel_l2(og[:, s0:s1], ro[:, s0:s1]) <= BARS[mode]
