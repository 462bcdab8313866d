"""Seeded random configurations of the range, packed-batch, paged-prefill and decode entry
points against the fp64 oracle on the same inputs: head counts and group sizes, head
dimensions, sequence and chunk lengths, key windows, query offsets, scale blocks, page
sizes, key splits, softmax scales and precisions drawn per case, so that combinations the
fixed-shape tests do not name are covered too. Each case prints its configuration first.

Bars as in the fixed-shape tests (relative L2 over the rows that see a key: FP8 exact and
lean 3e-2, BF16 5e-3; log-sum-exp within ln(1 + 2^-4), 0.1 and 1e-3). A case whose rows
that see a key number fewer than 64 is held to twice the bar: an L2 error over a handful
of rows is a small sample of the per-row error, whose spread the bars do not cover.
Rows that see no key must hold exactly 0 with LSE = -inf; rows of no sequence must keep
the sentinel the test wrote.

The quantizer's cases (head dimension, scale block, length, input type, rotation, value
distribution and magnitude drawn per case) are held to the quantizer tests' bars: without
rotation codes and scales equal the oracle's bit for bit; with it every code is a correct
rounding of the exactly rotated value over the kernel's scale, and every scale the least
power of two that holds its block's rotated absmax."""

import math

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from oracle import (dequantize_blocks, e4m3_decode, hadamard_rotate, paged_attention, quantize_blocks,
                    varlen_attention, window_attention)
from tests.paths import bf16_from_f64, rel_l2, rotation_noise, to_dev
from tests.test_gpu_decode import Decode
from tests.test_gpu_paged import Paged
from tests.test_gpu_varlen import SENTINEL, _inside, _packed, _run
from workloads import custom, generate

pytestmark = pytest.mark.gpu

BARS = {"fp8": 3e-2, "lean": 3e-2, "bf16": 5e-3}
LSE_TOL = {"fp8": math.log(1 + 2 ** -4), "lean": 0.1, "bf16": 1e-3}
MODES = ["bf16", "fp8", "lean"]


def _case(*a):
    print("case:", *a, flush=True)


def _heads(rng):
    Hkv = int(rng.integers(1, 4))
    return Hkv * int(rng.choice([1, 2, 3, 4])), Hkv


def _check(mode, o, lse, ro, rl, rows_seen):
    """o, lse and the oracle's ro, rl over the same rows (any leading shape); rows_seen
    counts the rows that see a key."""
    seen = np.isfinite(rl)
    assert np.array_equal(seen, np.isfinite(lse))
    assert np.all(o[~seen] == 0.0) and np.all(lse[~seen] == -np.inf)
    if not seen.any():
        return
    bar = BARS[mode] * (1 if rows_seen >= 64 else 2)
    err = rel_l2(o[seen], ro[seen])
    print(f"{mode} rel-L2 {err:.3e} over {rows_seen} rows (bar {bar:.0e})")
    assert err <= bar
    assert np.abs(lse[seen] - rl[seen]).max() < LSE_TOL[mode]


@pytest.mark.parametrize("seed", range(16))
def test_random_range_call(seed):
    rng = np.random.default_rng([1201, seed])
    mode = MODES[seed % 3]
    B = int(rng.integers(1, 3))
    Hq, Hkv = _heads(rng)
    Dqk, Dv = int(rng.choice([128, 192])), 128
    block = int(rng.choice([64, 128]))
    Skv = int(rng.integers(1, 700))
    k_begin = 64 * int(rng.integers(0, (Skv - 1) // 64 + 1))
    k_end = int(rng.integers(k_begin + 1, Skv + 1))
    Sq = int(rng.integers(1, 520))
    q_offset = int(rng.integers(0, 900))
    tau = 2.0 ** float(rng.uniform(-1, 1)) / math.sqrt(Dqk)
    _case(mode, dict(B=B, Hq=Hq, Hkv=Hkv, Dqk=Dqk, block=block, Sq=Sq, Skv=Skv, q_offset=q_offset,
                     window=(k_begin, k_end), tau=tau))
    q, _, _ = generate(custom(B, Hq, Hq, Sq, Dqk, Dv, wid=1210), seed=seed)
    _, k, v = generate(custom(B, Hkv, Hkv, Skv, Dqk, Dv, wid=1211), seed=seed)
    if mode == "bf16":
        t = [to_dev(x).to(torch.bfloat16) for x in (q, k, v)]
        o, lse = zy.attn_fwd_bf16_range(*t, q_offset, k_begin, k_end, tau, return_lse=True)
        deq = [x.float().cpu().numpy().astype(np.float64) for x in t]
    else:
        parts = [zy.quantize_fp8(to_dev(x), block) for x in (q, k, v)]
        o, lse = zy.attn_fwd_fp8_range(*[p[0] for p in parts], *[p[1] for p in parts], block, q_offset, k_begin,
                                       k_end, tau, return_lse=True, lean=mode == "lean")
        deq = [dequantize_blocks(c.cpu().numpy(), s.cpu().numpy(), block) for c, s in parts]
    torch.cuda.synchronize()
    ro, rl = window_attention(*deq, tau, q_offset=q_offset, k_begin=k_begin, k_end=k_end)
    rows_seen = int(np.isfinite(rl).sum())
    _check(mode, bf16_from_f64(o), lse.cpu().numpy().astype(np.float64), ro, rl, rows_seen)


@pytest.mark.parametrize("seed", range(8))
def test_random_packed_batch(seed):
    rng = np.random.default_rng([1202, seed])
    mode = MODES[seed % 3]
    Hq, Hkv = _heads(rng)
    Dqk, Dv = int(rng.choice([128, 192])), 128
    block = int(rng.choice([64, 128]))
    lengths = [int(x) for x in rng.integers(0, 500, size=int(rng.integers(1, 6)))]
    lengths[int(rng.integers(0, len(lengths)))] = max(1, lengths[0])  # at least one token
    tail = int(rng.integers(0, 70))
    _case(mode, dict(Hq=Hq, Hkv=Hkv, Dqk=Dqk, block=block, lengths=lengths, tail=tail))
    cu, q, k, v, T = _packed(lengths, tail, Hq, Hkv, Dqk, Dv, seed=100 + seed)
    max_seqlen = max(1, int(np.max(np.diff(cu))))
    o, lse, deq, _ = _run(mode, q, k, v, cu, max_seqlen, block)
    ro, rl = varlen_attention(deq[0], deq[1], deq[2], 1 / math.sqrt(Dqk), cu)
    inside = _inside(cu, T)
    og, lg = bf16_from_f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.all(og[:, ~inside] == SENTINEL) and np.all(lg[:, ~inside] == SENTINEL)
    _check(mode, og[:, inside], lg[:, inside], ro[:, inside], rl[:, inside], int(inside.sum()) * Hq)


@pytest.mark.parametrize("seed", range(8))
def test_random_paged_prefill(seed):
    rng = np.random.default_rng([1203, seed])
    mode = MODES[seed % 3]
    Hq, Hkv = _heads(rng)
    Dqk, Dv = int(rng.choice([128, 192])), 128
    P = int(rng.choice([64, 128, 256]))
    block = 64 if P == 64 else int(rng.choice([64, 128]))
    n = int(rng.integers(1, 5))
    chunks = [int(x) for x in rng.integers(0, 300, size=n)]
    kv = [c + int(rng.integers(0 if c else 1, 800)) for c in chunks]
    _case(mode, dict(Hq=Hq, Hkv=Hkv, Dqk=Dqk, P=P, block=block, kv_lens=kv, chunks=chunks))
    b = Paged(kv, chunks, P, Hq, Hkv, Dqk, Dv, seed=200 + seed)
    o, lse, deq, _ = b.run(mode, block=block)
    ro, rl = paged_attention(deq[0], deq[1], deq[2], 1 / math.sqrt(Dqk), b.cu, b.kv_lens, b.table)
    inside = b.inside()
    og, lg = bf16_from_f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.all(og[:, ~inside] == SENTINEL) and np.all(lg[:, ~inside] == SENTINEL)
    _check(mode, og[:, inside], lg[:, inside], ro[:, inside], rl[:, inside], int(inside.sum()) * Hq)


@pytest.mark.parametrize("seed", range(8))
def test_random_decode(seed):
    rng = np.random.default_rng([1204, seed])
    mode = MODES[seed % 3]
    Hkv = int(rng.integers(1, 4))
    Hq = Hkv * int(rng.choice([1, 4, 8, 16]))
    Dqk, Dv = int(rng.choice([128, 192])), 128
    P = int(rng.choice([64, 128, 256]))
    block = 64 if P == 64 else int(rng.choice([64, 128]))
    kv = [int(x) for x in rng.integers(1, 3000, size=int(rng.integers(1, 7)))]
    split = None if rng.integers(0, 2) else 64 * int(rng.integers(1, 20))
    _case(mode, dict(Hq=Hq, Hkv=Hkv, Dqk=Dqk, P=P, block=block, kv_lens=kv, split_keys=split))
    d = Decode(kv, P, Hq, Hkv, Dqk, Dv, seed=300 + seed)
    og, lg, deq = d.run(mode, block=block, split_keys=split)
    ro, rl = d.oracle(deq, 1 / math.sqrt(Dqk))
    _check(mode, og, lg, ro, rl, len(kv) * Hq)


@pytest.mark.parametrize("seed", range(12))
def test_random_quantize(seed):
    rng = np.random.default_rng([1205, seed])
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 6))
    D, block = int(rng.choice([128, 192])), int(rng.choice([64, 128]))
    S = int(rng.integers(1, 700))
    bf16, had = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    dist = str(rng.choice(["gaussian", "activation"]))
    mag = 2.0 ** float(rng.uniform(-20, 20))
    _case(dict(B=B, H=H, D=D, block=block, S=S, bf16=bf16, hadamard=had, dist=dist, magnitude=mag))
    x, _, _ = generate(custom(B, H, H, S, D, 128, dist=dist, wid=1220 + seed), seed=seed)
    xt = torch.from_numpy((x * np.float32(mag)).astype(np.float32))
    if bf16:
        xt = xt.to(torch.bfloat16)
    xr = xt.float().numpy()  # the values the kernel reads
    codes, scales = zy.quantize_fp8(xt.to("cuda"), block, had)
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    if not had:
        rc, rs = quantize_blocks(xr, block)
        assert np.array_equal(scales, rs) and np.array_equal(codes, rc)
        return
    y = hadamard_rotate(xr)  # exact rotation (float64)
    m, _ = np.frexp(scales.astype(np.float64))
    assert np.all(m == 0.5)
    t = y / np.repeat(scales.astype(np.float64), block, axis=2)[:, :, :S, None]
    err = np.abs(e4m3_decode(codes) - t)
    half_ulp = np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10)
    noise = rotation_noise(xr, scales, block)  # the kernel's float32 rotation error, in code units
    assert np.all(err <= half_ulp + noise * (1 + 2.0 ** -4) + np.abs(t) * 2.0 ** -20)
    for j in range(scales.shape[2]):
        r = np.abs(y[:, :, block * j:block * (j + 1)]).max(axis=(2, 3)) / scales[:, :, j]
        assert np.all(r <= 448 * (1 + 1e-6)) and np.all(r > 224 * (1 - 1e-6))
