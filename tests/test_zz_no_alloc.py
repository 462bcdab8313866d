"""The allocation-free decode (zyfa_attn_decode_fp8_paged_noalloc), through the C ABI,
against the decode entry point that takes a caller's workspace.

Both run the same kernels with the same key splits, so their outputs and log-sum-exps are
compared bit for bit: two calls in a row (the second smaller, reusing the library's scratch
array), a one-split call (no scratch needed), lean probabilities, and a request beyond the
scratch array's 8 MiB (rejected before any device work). The allocation-free calls write
into outputs the test allocates beforehand."""

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from fp8_causal_prefill_amd import _lib
from tests.paths import to_dev
from workloads import custom, generate, page_table, scatter_pages

pytestmark = pytest.mark.gpu


def _case(*a):
    print("case:", *a, flush=True)


def _decode_inputs(kv_lens, P, Hq, Hkv, D, block, seed):
    """FP8 decode operands: B sequences in a shuffled page cache, one query per sequence and
    query head (one scale per KV group)."""
    B = len(kv_lens)
    table, num_pages = page_table(kv_lens, P, seed)
    rng = np.random.default_rng([960, seed])
    k = rng.standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    v = rng.standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    for i, n in enumerate(kv_lens):
        _, kk, vv = generate(custom(1, Hkv, Hkv, n, D, D, wid=961 + i), seed=seed)
        scatter_pages(k, table[i], kk[0])
        scatter_pages(v, table[i], vv[0])
    q, _, _ = generate(custom(1, B, B, Hq, D, D, wid=970), seed=seed)
    g = Hq // Hkv
    qc, qs = zy.quantize_fp8(to_dev(q[0]).reshape(B, Hkv, g, D), block)
    kc, ks = zy.quantize_fp8(to_dev(k), block)
    vc, vs = zy.quantize_fp8(to_dev(v), block)
    return (qc.reshape(B, Hq, D), kc, vc, qs, ks, vs, torch.from_numpy(np.array(kv_lens, dtype=np.int32)).cuda(),
            torch.from_numpy(table).cuda())


def _both(ops, block, max_kv_len, split_keys, lean=False):
    qc, kc, vc, qs, ks, vs, kvl, bt = ops
    B, Hq, D = qc.shape
    o_ref, l_ref = zy.attn_decode_fp8_paged(qc, kc, vc, qs, ks, vs, block, kvl, bt, max_kv_len, split_keys=split_keys,
                                            return_lse=True, lean=lean)
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    zy.attn_decode_fp8_paged_noalloc(qc, kc, vc, qs, ks, vs, block, kvl, bt, max_kv_len, o, lse,
                                     split_keys=split_keys, lean=lean)
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref


def test_noalloc_decode_equals_workspace_decode_twice():
    Hq, Hkv, D, P, block = 8, 2, 128, 128, 64
    big = [1, 65, 700, 1500, 2048]
    _case("noalloc first call", big)
    ops1 = _decode_inputs(big, P, Hq, Hkv, D, block, seed=1)
    o, lse, o_ref, l_ref = _both(ops1, block, max(big), 128)  # 16 splits of the longest sequence
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    assert torch.all(torch.isfinite(o.float()))
    small = [33, 400, 900]
    _case("noalloc second, smaller call", small)
    ops2 = _decode_inputs(small, P, Hq, Hkv, D, block, seed=2)
    o2, lse2, o2_ref, l2_ref = _both(ops2, block, max(small), 64)  # 15 splits
    assert torch.equal(o2, o2_ref) and torch.equal(lse2, l2_ref)
    _case("noalloc one split and lean")
    o3, lse3, o3_ref, l3_ref = _both(ops2, block, max(small), 1024)  # one split: no scratch
    assert torch.equal(o3, o3_ref) and torch.equal(lse3, l3_ref)
    o4, lse4, o4_ref, l4_ref = _both(ops1, block, max(big), 256, lean=True)
    assert torch.equal(o4, o4_ref) and torch.equal(lse4, l4_ref)


def test_noalloc_decode_on_a_side_stream():
    # a stream other than the null stream: the library finds the scratch array of the
    # stream's device from the stream itself
    Hq, Hkv, D, P, block = 8, 2, 128, 128, 64
    lens = [70, 1300, 2000]
    _case("noalloc on a side stream", lens)
    ops = _decode_inputs(lens, P, Hq, Hkv, D, block, seed=4)
    o_ref, lse_ref, _, _ = _both(ops, block, max(lens), 128)
    side = torch.cuda.Stream()  # (default priority)
    side.wait_stream(torch.cuda.current_stream())
    qc, kc, vc, qs, ks, vs, kvl, bt = ops
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(lse_ref)
    with torch.cuda.stream(side):
        zy.attn_decode_fp8_paged_noalloc(qc, kc, vc, qs, ks, vs, block, kvl, bt, max(lens), o, lse, split_keys=128)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_noalloc_decode_rejects_requests_beyond_its_scratch():
    Hq, Hkv, D, P, block = 64, 8, 128, 128, 64
    _case("noalloc too large")
    ops = _decode_inputs([100, 200], P, Hq, Hkv, D, block, seed=3)
    qc, kc, vc, qs, ks, vs, kvl, bt = ops
    o = torch.empty((2, Hq, D), dtype=torch.bfloat16, device="cuda")
    max_kv = 1 << 20  # a bound of 2^20 keys in splits of 64: 16384 splits of 128 rows
    bt_big = torch.zeros((2, max_kv // P), dtype=torch.int32, device="cuda")
    need = zy.load().zyfa_attn_decode_workspace_bytes(2, Hq, D, max_kv, 64)
    assert need > zy.NOALLOC_SCRATCH_BYTES
    with pytest.raises(_lib.ZyfaError) as e:
        zy.attn_decode_fp8_paged_noalloc(qc, kc, vc, qs, ks, vs, block, kvl, bt_big, max_kv, o, split_keys=64)
    assert e.value.status == _lib.ERR_UNSUPPORTED
