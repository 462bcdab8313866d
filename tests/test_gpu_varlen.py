"""GPU attention over a packed batch of sequences of different lengths, through the C ABI,
against the fp64 oracle on the same inputs.

Bars as for the whole-sequence calls (relative L2 over the tokens of all sequences:
BF16 <= 5e-3, FP8 <= 3e-2, exact and lean). Beyond the bars: the real tokens of a sequence
padded at its end match the oracle on the unpadded sequence; every sequence equals a plain
call on that sequence alone bit for bit (same codes and scales); tokens after the last
sequence keep what the output held; a sequence whose cu_seqlens entries break the rules is
left unwritten while the others are computed.
"""

import math

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from oracle import dequantize_blocks, varlen_attention
from tests.paths import bf16_from_f64, rel_l2, to_dev
from workloads import custom, generate

pytestmark = pytest.mark.gpu

BARS = {"fp8": 3e-2, "lean": 3e-2, "bf16": 5e-3}
SENTINEL = 7.0


def _case(*a):
    print("case:", *a, flush=True)


def _packed(lengths, tail, Hq, Hkv, Dqk, Dv, seed):
    """Sequences of the given lengths packed with every start a multiple of 64: each but the
    last padded at its end to a multiple of 64 (padding that the sequence's own tokens never
    see: it follows them); `tail` tokens after the last sequence belong to none. Returns
    (cu_seqlens, q, k, v [H, T, D] float32, T, real lengths)."""
    cu = [0]
    for i, n in enumerate(lengths):
        cu.append(cu[-1] + (n if i == len(lengths) - 1 else -(-n // 64) * 64))
    T = cu[-1] + tail
    q, k, v = generate(custom(1, Hq, Hkv, T, Dqk, Dv, wid=900), seed=seed)
    return np.array(cu, dtype=np.int32), q[0], k[0], v[0], T


def _run(mode, q, k, v, cu, max_seqlen, block):
    Hq, T, _ = q.shape
    o = torch.full((Hq, T, v.shape[2]), SENTINEL, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((Hq, T), SENTINEL, dtype=torch.float32, device="cuda")
    cut = torch.from_numpy(cu).cuda()
    if mode == "bf16":
        t = [to_dev(x).to(torch.bfloat16) for x in (q, k, v)]
        zy.attn_fwd_bf16_varlen(*t, cut, max_seqlen, o=o, lse=lse)
        deq = [x.float().cpu().numpy().astype(np.float64) for x in t]
        parts = t
    else:
        parts = [zy.quantize_fp8(to_dev(x)[None], block) for x in (q, k, v)]
        c = [p[0][0] for p in parts]
        s = [p[1][0] for p in parts]
        zy.attn_fwd_fp8_varlen(*c, *s, block, cut, max_seqlen, o=o, lse=lse, lean=mode == "lean")
        deq = [dequantize_blocks(p[0].cpu().numpy(), p[1].cpu().numpy(), block)[0] for p in parts]
        parts = (c, s)
    torch.cuda.synchronize()
    return o, lse, deq, parts


def _inside(cu, T):
    m = np.zeros(T, dtype=bool)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        m[s0:s1] = True
    return m


@pytest.mark.parametrize("mode", ["bf16", "fp8", "lean"])
@pytest.mark.parametrize("shape", [(4, 2, 128, 128), (2, 2, 192, 128)])
def test_varlen_against_oracle(mode, shape):
    Hq, Hkv, Dqk, Dv = shape
    lengths = [300, 0, 64, 1000, 129, 1]
    _case(mode, shape, lengths)
    cu, q, k, v, T = _packed(lengths, 37, Hq, Hkv, Dqk, Dv, seed=1)
    max_seqlen = int(np.max(np.diff(cu)))
    o, lse, deq, _ = _run(mode, q, k, v, cu, max_seqlen, 128)
    tau = 1 / math.sqrt(Dqk)
    ro, rl = varlen_attention(deq[0], deq[1], deq[2], tau, cu)
    inside = _inside(cu, T)
    og, lg = bf16_from_f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.all(og[:, ~inside] == SENTINEL) and np.all(lg[:, ~inside] == SENTINEL)
    err = rel_l2(og[:, inside], ro[:, inside])
    print(f"{mode} varlen rel-L2 {err:.3e}")
    assert err <= BARS[mode]
    d = np.abs(lg[:, inside] - rl[:, inside])
    assert d.max() < (1e-3 if mode == "bf16" else (math.log(1 + 2 ** -4) if mode == "fp8" else 0.1))
    # the padding after a sequence is invisible to its real tokens: they match the oracle
    # on the unpadded sequences
    for a, n in zip(cu[:-1], lengths):
        if n:
            r1, _ = varlen_attention(deq[0], deq[1], deq[2], tau, [a, a + n])
            assert np.allclose(r1[:, a:a + n], ro[:, a:a + n], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["bf16", "fp8"])
def test_varlen_equals_plain_calls_per_sequence(mode):
    Hq, Hkv, D = 4, 1, 128
    lengths = [257, 64, 700, 3]
    _case(mode, "per-sequence", lengths)
    cu, q, k, v, T = _packed(lengths, 20, Hq, Hkv, D, D, seed=2)
    o, lse, _, parts = _run(mode, q, k, v, cu, int(np.max(np.diff(cu))), 64)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        if mode == "bf16":
            t = [x[None, :, s0:s1].clone() for x in parts]
            op, lp = zy.attn_fwd_bf16(*t, return_lse=True)
        else:
            c, s = parts
            # (clones: a slice of a one-head tensor is a contiguous view that keeps the
            # slice's offset, while the library wants 16-byte aligned pointers)
            cs = [x[None, :, s0:s1].clone() for x in c]
            ss = [x[None, :, s0 // 64:-(-s1 // 64)].clone() for x in s]
            op, lp = zy.attn_fwd_fp8(*cs, *ss, 64, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(op[0], o[:, s0:s1]) and torch.equal(lp[0], lse[:, s0:s1])


@pytest.mark.parametrize("mode", ["bf16", "fp8"])
def test_varlen_malformed_entry_leaves_its_sequence_unwritten(mode):
    Hq, Hkv, D = 2, 2, 128
    lengths = [200, 300, 150]
    _case(mode, "malformed", lengths)
    cu, q, k, v, T = _packed(lengths, 10, Hq, Hkv, D, D, seed=3)
    bad = cu.copy()
    bad[1] += 5  # the second sequence starts off the key tile (and the first ends later)
    o, lse, deq, _ = _run(mode, q, k, v, bad, int(np.max(np.diff(bad))), 128)
    og = bf16_from_f64(o)
    s0, s1 = bad[1], bad[2]
    assert np.all(og[:, s0:s1] == SENTINEL) and np.all(lse[:, s0:s1].cpu().numpy() == SENTINEL)
    ro, _ = varlen_attention(deq[0], deq[1], deq[2], 1 / math.sqrt(D), bad)
    for a, b in ((bad[0], bad[1]), (bad[2], bad[3])):
        assert rel_l2(og[:, a:b], ro[:, a:b]) <= BARS[mode]
