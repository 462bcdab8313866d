"""Parity at the full workload sizes (4K-32K tokens), in the launch configuration the
benchmark times, on rows the fp64 oracle computes one by one.

For each workload the GPU quantizes Q, K and V (with the Hadamard rotation of Q and K
for the activation-like workload's rotated variant) and runs the FP8 kernel (exact and
lean probabilities) and the BF16 kernel on the full tensors. The oracle then evaluates,
from the very codes and scales the kernel read (the quantizer itself is checked bit for
bit against the oracle elsewhere), two heads at:

* the first 256 query rows, which carry most of the whole-tensor norm (the output of
  row i is an average over i + 1 keys): rel-L2 over them must meet the bar;
* 24 rows spread over the rest of the sequence (seeded): the root-mean-square of their
  per-row relative errors must meet the same bar, and no row may exceed twice it.
"""

import math

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from oracle import causal_attention, dequantize_blocks
from tests.paths import bf16_from_f64, oracle_bf16
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu

BARS = {"fp8": 3e-2, "lean": 3e-2, "bf16": 5e-3}


def _late_rows(S, n=24, seed=0):
    rng = np.random.default_rng([4242, S, seed])
    return np.unique(np.concatenate([rng.choice(np.arange(256, S), n - 1, replace=False), [S - 1]]))


def _check(name, got_heads, ref_heads, rows_early, rows_late, bar):
    """got_heads / ref_heads: per head, [rows, Dv] float64 for early then late rows."""
    ne = len(rows_early)
    ge = np.concatenate([g[:ne] for g in got_heads])
    re_ = np.concatenate([r[:ne] for r in ref_heads])
    early = np.linalg.norm(ge - re_) / np.linalg.norm(re_)
    per_row = np.concatenate([np.linalg.norm(g[ne:] - r[ne:], axis=1) / np.linalg.norm(r[ne:], axis=1)
                              for g, r in zip(got_heads, ref_heads)])
    late_rms = float(np.sqrt(np.mean(per_row ** 2)))
    print(f"{name}: early rows rel-L2 {early:.3e}, late rows rms {late_rms:.3e}, max {per_row.max():.3e}", flush=True)
    assert early <= bar
    assert late_rms <= bar
    assert per_row.max() <= 2 * bar


@pytest.mark.parametrize("wname,hadamard", [("mha4k", False), ("gqa32k", False), ("mla32k", False),
                                             ("act16k", False), ("act16k", True)])
def test_full_size_fp8_exact_and_lean(wname, hadamard):
    w = WORKLOADS[wname]
    print(f"case: {wname} hadamard={hadamard}", flush=True)
    q, k, v = generate(w, seed=0)
    dev = "cuda"
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    del q, k, v
    qc, qs = zy.quantize_fp8(qd, w.scale_block, hadamard)
    kc, ks = zy.quantize_fp8(kd, w.scale_block, hadamard)
    vc, vs = zy.quantize_fp8(vd, w.scale_block, False)
    del qd, kd, vd
    outs = {}
    for mode in ("fp8", "lean"):
        o, _ = zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, w.scale_block, w.softmax_scale, lean=(mode == "lean"))
        outs[mode] = o
    torch.cuda.synchronize()
    rows_e = np.arange(256)
    rows_l = _late_rows(w.S)
    rows = np.concatenate([rows_e, rows_l])
    group = w.Hq // w.Hkv
    ref_heads, got = [], {m: [] for m in outs}
    for hq in (0, w.Hq - 1):
        hk = hq // group
        deq = [dequantize_blocks(c[0:1, h:h + 1].cpu().numpy(), s[0:1, h:h + 1].cpu().numpy(), w.scale_block)
               for c, s, h in ((qc, qs, hq), (kc, ks, hk), (vc, vs, hk))]
        ro, _ = causal_attention(deq[0], deq[1], deq[2], w.softmax_scale, rows=rows)
        ref_heads.append(ro[0, 0])
        for m, o in outs.items():
            got[m].append(bf16_from_f64(o[0, hq, torch.from_numpy(rows).to(dev)]))
    for m in outs:
        _check(f"{wname} {m}", got[m], ref_heads, rows_e, rows_l, BARS[m])


@pytest.mark.parametrize("wname", ["mha4k", "gqa32k", "mla32k", "act16k"])
def test_full_size_bf16(wname):
    w = WORKLOADS[wname]
    print(f"case: {wname} bf16", flush=True)
    q, k, v = generate(w, seed=0)
    dev = "cuda"
    tb = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
    qb, kb, vb = tb(q), tb(k), tb(v)
    o, _ = zy.attn_fwd_bf16(qb, kb, vb, w.softmax_scale)
    torch.cuda.synchronize()
    rows_e = np.arange(256)
    rows_l = _late_rows(w.S, seed=1)
    rows = np.concatenate([rows_e, rows_l])
    group = w.Hq // w.Hkv
    ref_heads, got_heads = [], []
    for hq in (0, w.Hq - 1):
        hk = hq // group
        ro, _, _ = oracle_bf16(q[0:1, hq:hq + 1], k[0:1, hk:hk + 1], v[0:1, hk:hk + 1], w.softmax_scale, rows=rows)
        ref_heads.append(ro[0, 0])
        got_heads.append(bf16_from_f64(o[0, hq, torch.from_numpy(rows).to(dev)]))
    _check(f"{wname} bf16", got_heads, ref_heads, rows_e, rows_l, BARS["bf16"])


def test_full_size_range_chunk_and_split_kv():
    """The range measurements of the benchmark at the headline shape (32K GQA, FP8 exact):
    the second half of the sequence as a chunk against its prefix, and the keys split into
    [0, S/2) and [S/2, S) merged by zyfa_attn_merge. Checked on sampled rows of two heads
    against the oracle (the chunk also bit for bit against the full call's rows)."""
    from oracle import merge_partials, window_attention
    w = WORKLOADS["gqa32k"]
    print("case: gqa32k range chunk + split-KV", flush=True)
    q, k, v = generate(w, seed=0)
    dev = "cuda"
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    del q, k, v
    blk, S = w.scale_block, w.S
    qc, qs = zy.quantize_fp8(qd, blk)
    kc, ks = zy.quantize_fp8(kd, blk)
    vc, vs = zy.quantize_fp8(vd, blk)
    del qd, kd, vd
    half = S // 2
    o_full, l_full = zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, w.softmax_scale, return_lse=True)
    o_chunk, l_chunk = zy.attn_fwd_fp8_range(qc[:, :, half:].contiguous(), kc, vc, qs[:, :, half // blk:].contiguous(),
                                             ks, vs, blk, half, 0, S, w.softmax_scale, return_lse=True)
    parts = [zy.attn_fwd_fp8_range(qc, kc, vc, qs, ks, vs, blk, 0, lo, hi, w.softmax_scale, return_lse=True)
             for lo, hi in ((0, half), (half, S))]
    o_m, l_m = zy.attn_merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]), return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_chunk, o_full[:, :, half:]) and torch.equal(l_chunk, l_full[:, :, half:])
    # chunk rows: the first 256 of the chunk and 24 spread over it; merged output: the
    # first 256 rows of the sequence, which see only the first window, and 24 spread
    rows_c_e = np.arange(256)
    rows_c_l = _late_rows(S - half, seed=2)
    rows_m_l = _late_rows(S, seed=3)
    group = w.Hq // w.Hkv
    ref_c, got_c, ref_m, got_m = [], [], [], []
    for hq in (0, w.Hq - 1):
        hk = hq // group
        deq = [dequantize_blocks(c[0:1, h:h + 1].cpu().numpy(), s[0:1, h:h + 1].cpu().numpy(), blk)
               for c, s, h in ((qc, qs, hq), (kc, ks, hk), (vc, vs, hk))]
        rows_c = np.concatenate([rows_c_e, rows_c_l])
        rc, _ = window_attention(deq[0][:, :, half:], deq[1], deq[2], w.softmax_scale, q_offset=half, rows=rows_c)
        ref_c.append(rc[0, 0])
        got_c.append(bf16_from_f64(o_chunk[0, hq, torch.from_numpy(rows_c).to(dev)]))
        rows_m = np.concatenate([np.arange(256), rows_m_l])
        pr = [window_attention(deq[0], deq[1], deq[2], w.softmax_scale, k_begin=lo, k_end=hi, rows=rows_m)
              for lo, hi in ((0, half), (half, S))]
        rm, _ = merge_partials(np.stack([p[0] for p in pr]), np.stack([p[1] for p in pr]))
        ref_m.append(rm[0, 0])
        got_m.append(bf16_from_f64(o_m[0, hq, torch.from_numpy(rows_m).to(dev)]))
    _check("gqa32k chunk", got_c, ref_c, rows_c_e, rows_c_l, BARS["fp8"])
    _check("gqa32k split-KV merged", got_m, ref_m, np.arange(256), rows_m_l, BARS["fp8"])


def test_full_size_varlen_batch():
    """The packed batch the benchmark times: the 32K GQA tensors read as [H, T, D] and split
    into sequences of 16384 .. 256 tokens (FP8 exact). Sampled rows of two heads against the
    oracle: the first 256 rows of the batch and 24 spread over it."""
    from oracle import varlen_attention
    import bench
    w = WORKLOADS["gqa32k"]
    print("case: gqa32k varlen batch", flush=True)
    q, k, v = generate(w, seed=0)
    dev = "cuda"
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    del q, k, v
    blk = w.scale_block
    qc, qs = zy.quantize_fp8(qd, blk)
    kc, ks = zy.quantize_fp8(kd, blk)
    vc, vs = zy.quantize_fp8(vd, blk)
    del qd, kd, vd
    lengths = bench.VARLEN_LENGTHS
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    o, _ = zy.attn_fwd_fp8_varlen(qc[0], kc[0], vc[0], qs[0], ks[0], vs[0], blk, torch.from_numpy(cu).to(dev),
                                  max(lengths), w.softmax_scale)
    torch.cuda.synchronize()
    rows_e = np.arange(256)
    rows_l = _late_rows(w.S, seed=4)
    rows = np.concatenate([rows_e, rows_l])
    group = w.Hq // w.Hkv
    ref_heads, got_heads = [], []
    for hq in (0, w.Hq - 1):
        hk = hq // group
        deq = [dequantize_blocks(c[0:1, h:h + 1].cpu().numpy(), s[0:1, h:h + 1].cpu().numpy(), blk)[0]
               for c, s, h in ((qc, qs, hq), (kc, ks, hk), (vc, vs, hk))]
        ro, _ = varlen_attention(deq[0], deq[1], deq[2], w.softmax_scale, cu, rows=rows)
        ref_heads.append(ro[0])
        got_heads.append(bf16_from_f64(o[hq, torch.from_numpy(rows).to(dev)]))
    _check("gqa32k varlen", got_heads, ref_heads, rows_e, rows_l, BARS["fp8"])


def test_full_size_paged_prefill():
    """The paged measurements of the benchmark: the 32K GQA keys and values in a shuffled
    cache of 128-token pages (FP8 exact), the whole sequence as one chunk and its second
    half as a chunk after a 16K cached prefix. Bit for bit against the plain and range calls
    on the contiguous tensors, and on sampled rows of two heads against the oracle on the
    pages it gathers through the block table."""
    from oracle import gather_pages, window_attention
    import bench
    w = WORKLOADS["gqa32k"]
    print("case: gqa32k paged prefill", flush=True)
    q, k, v = generate(w, seed=0)
    dev = "cuda"
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    del q, k, v
    blk, S = w.scale_block, w.S
    qc, qs = zy.quantize_fp8(qd, blk)
    kc, ks = zy.quantize_fp8(kd, blk)
    vc, vs = zy.quantize_fp8(vd, blk)
    del qd, kd, vd
    kp, vp, ksp, vsp, bt = bench.paged_cache(w, kc, vc, ks, vs, torch)
    kvl = torch.tensor([S], dtype=torch.int32, device=dev)
    half = S // 2
    o_w, l_w = zy.attn_fwd_fp8_paged(qc[0], kp, vp, qs[0], ksp, vsp, blk, torch.tensor([0, S], dtype=torch.int32,
                                     device=dev), kvl, bt, S, w.softmax_scale, return_lse=True)
    o_c, l_c = zy.attn_fwd_fp8_paged(qc[0, :, half:].contiguous(), kp, vp, qs[0, :, half // blk:].contiguous(), ksp,
                                     vsp, blk, torch.tensor([0, S - half], dtype=torch.int32, device=dev), kvl, bt,
                                     S - half, w.softmax_scale, return_lse=True)
    o_full, l_full = zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, blk, w.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_w, o_full[0]) and torch.equal(l_w, l_full[0])
    assert torch.equal(o_c, o_full[0, :, half:]) and torch.equal(l_c, l_full[0, :, half:])
    del o_full, l_full
    rows_e = np.arange(256)
    rows_l = _late_rows(S - half, seed=5)
    rows = np.concatenate([rows_e, rows_l])
    table = bt[0].cpu().numpy()
    group = w.Hq // w.Hkv
    ref_heads, got_heads = [], []
    for hq in (0, w.Hq - 1):
        hk = hq // group
        qq = dequantize_blocks(qc[0:1, hq:hq + 1].cpu().numpy(), qs[0:1, hq:hq + 1].cpu().numpy(), blk)
        kk, vv = (gather_pages(dequantize_blocks(c[:, hk:hk + 1].cpu().numpy(), s[:, hk:hk + 1].cpu().numpy(), blk),
                               table, S) for c, s in ((kp, ksp), (vp, vsp)))
        ro, _ = window_attention(qq[:, :, half:], kk[None], vv[None], w.softmax_scale, q_offset=half, rows=rows)
        ref_heads.append(ro[0, 0])
        got_heads.append(bf16_from_f64(o_c[hq, torch.from_numpy(rows).to(dev)]))
    _check("gqa32k paged chunk", got_heads, ref_heads, rows_e, rows_l, BARS["fp8"])


def test_full_size_decode_batch():
    """The decode measurement of the benchmark: 8 sequences of 32K keys in a shuffled page
    cache at the headline heads (FP8 exact, the split and merge the benchmark times). Every
    output against the oracle on the pages it gathers (one-token chunks at position
    32767)."""
    from oracle import gather_pages, window_attention
    import bench
    w = WORKLOADS["gqa32k"]
    print("case: gqa32k decode batch", flush=True)
    _, k, v = generate(w, seed=0)
    dev = "cuda"
    kd, vd = (torch.from_numpy(x).to(dev) for x in (k, v))
    del k, v
    blk, S = w.scale_block, w.S
    kc, ks = zy.quantize_fp8(kd, blk)
    vc, vs = zy.quantize_fp8(vd, blk)
    del kd, vd
    qc, qs, kp, vp, ksp, vsp, kvl, bt = bench.decode_setup(w, kc, vc, ks, vs, torch, zy)
    B = qc.shape[0]
    split = zy.decode_split_keys(B, w.Hkv, S)
    o, lse = zy.attn_decode_fp8_paged(qc, kp, vp, qs, ksp, vsp, blk, kvl, bt, S, w.softmax_scale, split_keys=split,
                                      return_lse=True)
    torch.cuda.synchronize()
    g = w.Hq // w.Hkv
    qq = dequantize_blocks(qc.reshape(B, w.Hkv, g, w.Dqk).cpu().numpy(), qs.cpu().numpy(), blk)  # [B, Hkv, g, D]
    table = bt.cpu().numpy()
    got, ref = [], []
    for b in (0, B - 1):
        # the sequence's pages, in table order, dequantized; then laid end to end
        pages = torch.from_numpy(table[b].astype(np.int64)).to(dev)
        for hk in range(w.Hkv):
            kk, vv = (dequantize_blocks(c[pages, hk:hk + 1].cpu().numpy(), s_[pages, hk:hk + 1].cpu().numpy(), blk)
                      for c, s_ in ((kp, ksp), (vp, vsp)))
            ident = np.arange(len(table[b]))
            kg, vg = gather_pages(kk, ident, S), gather_pages(vv, ident, S)  # [1, S, D]
            ro, _ = window_attention(qq[b, hk][None, :, None], kg[None], vg[None], w.softmax_scale, q_offset=S - 1)
            ref.append(ro[0, :, 0])
            got.append(bf16_from_f64(o[b, hk * g:(hk + 1) * g]))
    got, ref = np.stack(got), np.stack(ref)
    err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"gqa32k decode rel-L2 {err:.3e}")
    assert err <= BARS["fp8"]


def test_full_size_decode_batch_bf16():
    """The BF16 decode measurement of the benchmark: the same batch as the FP8 one in
    bfloat16, with the split size the benchmark uses for it; the outputs of two sequences
    against the oracle on the pages it gathers."""
    from oracle import gather_pages, window_attention
    import bench
    w = WORKLOADS["gqa32k"]
    print("case: gqa32k decode batch bf16", flush=True)
    _, k, v = generate(w, seed=0)
    dev = "cuda"
    kd, vd = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (k, v))
    del k, v
    S = w.S
    qb, _, kp, vp, _, _, kvl, bt = bench.decode_setup(w, kd, vd, None, None, torch, zy)
    del kd, vd
    B = qb.shape[0]
    split = zy.decode_split_keys(B, w.Hkv, S, 256)
    o, _ = zy.attn_decode_bf16_paged(qb, kp, vp, kvl, bt, S, w.softmax_scale, split_keys=split)
    torch.cuda.synchronize()
    g = w.Hq // w.Hkv
    qq = qb.float().cpu().numpy().astype(np.float64).reshape(B, w.Hkv, g, w.Dqk)
    table = bt.cpu().numpy()
    got, ref = [], []
    for b in (0, B - 1):
        pages = torch.from_numpy(table[b].astype(np.int64)).to(dev)
        ident = np.arange(len(table[b]))
        for hk in range(w.Hkv):
            kk, vv = (c[pages, hk:hk + 1].float().cpu().numpy().astype(np.float64) for c in (kp, vp))
            kg, vg = gather_pages(kk, ident, S), gather_pages(vv, ident, S)
            ro, _ = window_attention(qq[b, hk][None, :, None], kg[None], vg[None], w.softmax_scale, q_offset=S - 1)
            ref.append(ro[0, :, 0])
            got.append(bf16_from_f64(o[b, hk * g:(hk + 1) * g]))
    got, ref = np.stack(got), np.stack(ref)
    err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"gqa32k decode bf16 rel-L2 {err:.3e}")
    assert err <= BARS["bf16"]
