"""LDS poisoning (environment variable ZYFA_LDS_POISON): every attention kernel, run with
its LDS filled with all-ones bytes before its first tile copy, gives bit for bit the
output of the normal run.

All-ones bytes are a NaN in e4m3 and in bfloat16, so a kernel that read any LDS byte its
tile copies had not written (a stale buffer, a row past a ragged tile, a buffer read
before its copy landed) would carry the NaN into O or the log-sum-exp. Covered: the
whole-sequence calls at both head shapes in all three modes (ragged lengths), a chunk
against a key window, a packed batch, prefill against a paged cache, and decode on the
one-wave (FP8) and eight-wave (BF16) workgroups with several key splits.
"""

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from tests.paths import to_dev
from tests.test_gpu_decode import Decode
from tests.test_gpu_paged import Paged
from workloads import custom, generate

pytestmark = pytest.mark.gpu


def _case(*a):
    print("case:", *a, flush=True)


def _same_with_poison(monkeypatch, fn):
    """fn() -> tensors or arrays; equal bit for bit with and without the poison (NaN never
    equals itself, so a poisoned byte that reached an output fails the comparison)."""
    monkeypatch.delenv("ZYFA_LDS_POISON", raising=False)
    ref = [t.clone() if torch.is_tensor(t) else np.copy(t) for t in fn()]
    torch.cuda.synchronize()
    monkeypatch.setenv("ZYFA_LDS_POISON", "1")
    got = fn()
    torch.cuda.synchronize()
    monkeypatch.delenv("ZYFA_LDS_POISON")
    for a, b in zip(ref, got):
        if torch.is_tensor(a):
            assert not torch.isnan(a.float()).any()
            assert torch.equal(a, b)
        else:
            assert not np.isnan(a).any()
            assert np.array_equal(a, b)


def _inputs(Hq, Hkv, S, Dqk, wid, block=128):
    q, k, v = generate(custom(1, Hq, Hkv, S, Dqk, 128, wid=wid), seed=3)
    f8 = [zy.quantize_fp8(to_dev(x), block) for x in (q, k, v)]
    bf = [to_dev(x).to(torch.bfloat16) for x in (q, k, v)]
    return f8, bf


@pytest.mark.parametrize("Hq,Hkv,S,Dqk", [(4, 2, 1000, 128), (2, 2, 777, 192)])
def test_whole_sequence_calls(monkeypatch, Hq, Hkv, S, Dqk):
    f8, bf = _inputs(Hq, Hkv, S, Dqk, wid=980 + Dqk)
    (qc, qs), (kc, ks), (vc, vs) = f8
    for mode in ("fp8", "lean", "bf16"):
        _case(mode, Hq, Hkv, S, Dqk)
        if mode == "bf16":
            _same_with_poison(monkeypatch, lambda: zy.attn_fwd_bf16(*bf, return_lse=True))
        else:
            _same_with_poison(monkeypatch, lambda: zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, 128, return_lse=True,
                                                                  lean=mode == "lean"))


def test_chunk_against_key_window(monkeypatch):
    f8, bf = _inputs(4, 2, 1000, 128, wid=983)
    (qc, qs), (kc, ks), (vc, vs) = f8
    q2, qs2 = qc[:, :, 512:].contiguous(), qs[:, :, 4:].contiguous()
    _case("fp8 range q_offset 512, window [64, 1000)")
    _same_with_poison(monkeypatch, lambda: zy.attn_fwd_fp8_range(q2, kc, vc, qs2, ks, vs, 128, q_offset=512,
                                                                 k_begin=64, k_end=1000, return_lse=True))
    _case("bf16 range q_offset 512, window [64, 1000)")
    qb2 = bf[0][:, :, 512:].contiguous()
    _same_with_poison(monkeypatch, lambda: zy.attn_fwd_bf16_range(qb2, bf[1], bf[2], q_offset=512, k_begin=64,
                                                                  k_end=1000, return_lse=True))


def test_packed_batch(monkeypatch):
    lengths = [300, 64, 1000, 129]
    cu = [0]
    for i, n in enumerate(lengths):
        cu.append(cu[-1] + (n if i == len(lengths) - 1 else -(-n // 64) * 64))
    T = cu[-1] + 21
    f8, bf = _inputs(4, 2, T, 128, wid=984, block=64)
    (qc, qs), (kc, ks), (vc, vs) = f8
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    mx = int(np.max(np.diff(cu)))
    for mode in ("fp8", "lean"):
        _case(mode, "varlen", lengths)
        _same_with_poison(monkeypatch, lambda: zy.attn_fwd_fp8_varlen(qc[0], kc[0], vc[0], qs[0], ks[0], vs[0], 64,
                                                                      cud, mx, return_lse=True,
                                                                      lean=mode == "lean"))
    _case("bf16 varlen", lengths)
    _same_with_poison(monkeypatch, lambda: zy.attn_fwd_bf16_varlen(bf[0][0], bf[1][0], bf[2][0], cud, mx,
                                                                   return_lse=True))


@pytest.mark.parametrize("P", [64, 256])
def test_paged_prefill(monkeypatch, P):
    pg = Paged([700, 64, 1000], [200, 64, 333], P, 4, 2, 128, 128, seed=P)
    for mode in ("fp8", "lean", "bf16"):
        _case(mode, "paged prefill, page", P)
        _same_with_poison(monkeypatch, lambda: pg.run(mode)[:2])


@pytest.mark.parametrize("split_keys", [None, 128])
def test_decode(monkeypatch, split_keys):
    dec = Decode([700, 1, 1000, 129], 64, 8, 2, 128, 128, seed=5)
    for mode in ("fp8", "lean", "bf16"):
        _case(mode, "decode, split", split_keys)
        _same_with_poison(monkeypatch, lambda: dec.run(mode, split_keys=split_keys)[:2])
