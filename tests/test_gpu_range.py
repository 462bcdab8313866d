"""GPU range entry points (a chunk of query rows against a key window) and the merge of
partial results, through the C ABI, against the fp64 oracle on the same inputs.

Bars as for the whole-sequence calls: relative L2 over the output rows that see a key,
BF16 <= 5e-3, FP8 <= 3e-2 (exact and lean). Rows that see no key must be exactly 0 with
LSE = -inf. Beyond the bars:

* the range call over the whole sequence is the plain call, bit for bit;
* a chunk of rows at offset a, whose codes and scales are the full sequence's, returns
  exactly the full call's rows (each row's computation does not depend on the rows that
  share its workgroup);
* split-KV: windows over the keys, each checked against the oracle, merged on the GPU,
  match one pass over all keys (the oracle's causal attention);
* the merge kernel on given bf16 parts matches the oracle's merge of the same values to
  bfloat16 rounding (unit roundoff 2^-8).
"""

import math

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from oracle import causal_attention, dequantize_blocks, merge_partials, window_attention
from tests.paths import bf16_from_f64, rel_l2, to_dev
from workloads import custom, generate

pytestmark = pytest.mark.gpu

BARS = {"fp8": 3e-2, "lean": 3e-2, "bf16": 5e-3}


def _check_lse(mode, got, ref):
    """Log-sum-exp (natural log) of rows that see a key. An e4m3 rounding of a probability
    is off by at most 2^-4 of the block maximum's scale, so the row sum by at most a
    factor 1 + 2^-4; bfloat16 probabilities by far less. A lean code of a value in e4m3's
    normal range is off by at most 0.068 in log (once the kernel divides out the codes'
    common factor); with the block maximum scaled into [128, 256), only weights under
    2^-13 of it are subnormal (where the linear code is far off), and 64 of them sum to
    less than 2^-7 of it: a lean row is off by less than 0.1."""
    d = np.abs(got - ref)
    if mode == "lean":
        assert d.max() < 0.1 and math.sqrt(np.mean(d ** 2)) < 0.02
    else:
        assert d.max() < (math.log(1 + 2 ** -4) if mode == "fp8" else 1e-3)


def _case(*a):
    print("case:", *a, flush=True)


def _inputs(B, Hq, Hkv, S, Dqk, Dv, seed, wid=700):
    return generate(custom(B, Hq, Hkv, S, Dqk, Dv, wid=wid), seed=seed)


class Side:
    """One precision's GPU inputs and the dequantized values the kernel reads."""

    def __init__(self, mode, q, k, v, block=128):
        self.mode, self.block = mode, block
        if mode == "bf16":
            self.t = [to_dev(x).to(torch.bfloat16) for x in (q, k, v)]
            self.deq = [t.float().cpu().numpy().astype(np.float64) for t in self.t]
        else:
            parts = [zy.quantize_fp8(to_dev(x), block) for x in (q, k, v)]
            self.t = [p[0] for p in parts]
            self.s = [p[1] for p in parts]
            self.deq = [dequantize_blocks(c.cpu().numpy(), s.cpu().numpy(), block) for c, s in parts]

    def plain(self, scale):
        if self.mode == "bf16":
            return zy.attn_fwd_bf16(*self.t, scale, return_lse=True)
        return zy.attn_fwd_fp8(*self.t, *self.s, self.block, scale, return_lse=True, lean=self.mode == "lean")

    def range(self, scale, q_offset=0, k_begin=0, k_end=None, q_rows=None):
        q = self.t[0] if q_rows is None else self.t[0][:, :, q_rows[0]:q_rows[1]].contiguous()
        if self.mode == "bf16":
            return zy.attn_fwd_bf16_range(q, self.t[1], self.t[2], q_offset, k_begin, k_end, scale, return_lse=True)
        qs = self.s[0]
        if q_rows is not None:
            assert q_rows[0] % self.block == 0
            qs = qs[:, :, q_rows[0] // self.block:(q_rows[1] + self.block - 1) // self.block].contiguous()
        return zy.attn_fwd_fp8_range(q, self.t[1], self.t[2], qs, self.s[1], self.s[2], self.block, q_offset, k_begin,
                                     k_end, scale, return_lse=True, lean=self.mode == "lean")


def _np(o, lse):
    torch.cuda.synchronize()
    return bf16_from_f64(o), lse.cpu().numpy().astype(np.float64)


MODES = ["bf16", "fp8", "lean"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(1, 4, 2, 333, 128, 128), (1, 2, 2, 300, 192, 128)])
def test_whole_sequence_range_is_the_plain_call(mode, shape):
    B, Hq, Hkv, S, Dqk, Dv = shape
    _case(mode, shape)
    side = Side(mode, *_inputs(B, Hq, Hkv, S, Dqk, Dv, seed=1))
    o1, l1 = _np(*side.plain(1 / math.sqrt(Dqk)))
    o2, l2 = _np(*side.range(1 / math.sqrt(Dqk)))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("rows", [(256, 700), (128, 384), (512, 900)])
def test_chunk_of_rows_matches_full_call_and_oracle(mode, rows):
    B, Hq, Hkv, S, D = 1, 4, 2, 900, 128
    a, b = rows
    _case(mode, rows)
    side = Side(mode, *_inputs(B, Hq, Hkv, S, D, D, seed=2))
    tau = 1 / math.sqrt(D)
    o_full, l_full = _np(*side.plain(tau))
    o, l = _np(*side.range(tau, q_offset=a, k_end=b, q_rows=(a, b)))
    assert np.array_equal(o, o_full[:, :, a:b]) and np.array_equal(l, l_full[:, :, a:b])
    ro, rl = window_attention(side.deq[0][:, :, a:b], side.deq[1], side.deq[2], tau, q_offset=a, k_end=b)
    err = rel_l2(o, ro)
    print(f"{mode} chunk rel-L2 {err:.3e}")
    assert err <= BARS[mode]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("cfg", [
    # (B, Hq, Hkv, S, Dqk, scale block, window edges)
    (1, 4, 2, 1000, 128, 128, [0, 320, 1000]),
    (2, 4, 1, 700, 128, 64, [0, 64, 128, 512, 700]),
    (1, 2, 2, 600, 192, 128, [0, 192, 600]),
])
def test_split_kv_parts_and_merge(mode, cfg):
    B, Hq, Hkv, S, Dqk, block, edges = cfg
    _case(mode, cfg)
    side = Side(mode, *_inputs(B, Hq, Hkv, S, Dqk, 128, seed=3), block=block)
    tau = 1 / math.sqrt(Dqk)
    o_parts, l_parts = [], []
    for lo, hi in zip(edges[:-1], edges[1:]):
        o, l = side.range(tau, k_begin=lo, k_end=hi)
        on, ln = _np(o, l)
        ro, rl = window_attention(*side.deq, tau, k_begin=lo, k_end=hi)
        seen = np.isfinite(rl)
        assert np.array_equal(seen, np.isfinite(ln))
        assert np.all(on[~seen] == 0.0)
        err = rel_l2(on[seen], ro[seen])
        print(f"{mode} window [{lo}, {hi}) rel-L2 {err:.3e}")
        assert err <= BARS[mode]
        _check_lse(mode, ln[seen], rl[seen])
        o_parts.append(o)
        l_parts.append(l)
    om, lm = zy.attn_merge(torch.stack(o_parts), torch.stack(l_parts), return_lse=True)
    om, lm = _np(om, lm)
    ro, rl = causal_attention(*side.deq, tau)
    err = rel_l2(om, ro)
    print(f"{mode} merged rel-L2 {err:.3e}")
    assert err <= BARS[mode]
    _check_lse(mode, lm, rl)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("window", [(0, 100), (64, 100), (128, 1000), (0, 37)])
def test_window_ending_before_the_rows(mode, window):
    # every row (positions 0 .. 999) against a window that later rows see whole, ending
    # inside a key tile: the window's end is masked like the causal diagonal
    B, Hq, Hkv, S, D = 1, 2, 2, 1000, 128
    lo, hi = window
    _case(mode, window)
    side = Side(mode, *_inputs(B, Hq, Hkv, S, D, D, seed=6))
    tau = 1 / math.sqrt(D)
    o, l = _np(*side.range(tau, k_begin=lo, k_end=hi))
    ro, rl = window_attention(*side.deq, tau, k_begin=lo, k_end=hi)
    seen = np.isfinite(rl)
    assert np.array_equal(seen, np.isfinite(l)) and np.all(o[~seen] == 0.0)
    err = rel_l2(o[seen], ro[seen])
    print(f"{mode} rel-L2 {err:.3e}")
    assert err <= BARS[mode]
    _check_lse(mode, l[seen], rl[seen])


@pytest.mark.parametrize("mode", MODES)
def test_rows_and_workgroups_without_keys(mode):
    # query rows at positions 100 .. 899 against keys [640, 900): the first 540 rows see no
    # key, including two whole workgroups of 256 rows
    B, Hq, Hkv, Sq, Skv, D = 1, 2, 1, 800, 900, 128
    _case(mode, "empty rows")
    q, _, _ = _inputs(B, Hq, Hkv, Sq, D, D, seed=4)
    _, k, v = _inputs(B, Hkv, Hkv, Skv, D, D, seed=5)
    side = Side(mode, q, k, v)
    tau = 1 / math.sqrt(D)
    o, l = _np(*side.range(tau, q_offset=100, k_begin=640))
    ro, rl = window_attention(*side.deq, tau, q_offset=100, k_begin=640)
    empty = np.arange(Sq) + 100 < 640
    assert np.all(o[:, :, empty] == 0.0) and np.all(l[:, :, empty] == -np.inf)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l[:, :, ~empty]))
    err = rel_l2(o[:, :, ~empty], ro[:, :, ~empty])
    print(f"{mode} rel-L2 {err:.3e}")
    assert err <= BARS[mode]


@pytest.mark.parametrize("Dv", [64, 128, 256, 512])
@pytest.mark.parametrize("P", [1, 2, 5])
def test_merge_kernel_against_oracle(Dv, P):
    _case("merge", Dv, P)
    rng = np.random.default_rng([800, Dv, P])
    R = 3001
    o = rng.standard_normal((P, R, Dv)).astype(np.float32)
    lse = (rng.standard_normal((P, R)) * 6).astype(np.float32)
    lse[0, ::7] = -np.inf                # part 0 saw no key of some rows
    lse[:, 5] = -np.inf                  # no part saw row 5
    lse[:, 6] = 1.0e4                    # values far outside exp's range
    ob = torch.from_numpy(o).to(torch.bfloat16).cuda()
    lb = torch.from_numpy(lse).cuda()
    om, lm = zy.attn_merge(ob, lb, return_lse=True)
    om, lm = _np(om, lm)
    ro, rl = merge_partials(ob.float().cpu().numpy(), lse)
    assert np.all(om[5] == 0.0) and lm[5] == -np.inf
    err = rel_l2(om, ro)
    print(f"merge rel-L2 {err:.3e}")
    assert err <= 2.0 ** -8 + 1e-5  # bfloat16 rounding of the output
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lm))
    assert np.max(np.abs(lm[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin]))) <= 1e-6
