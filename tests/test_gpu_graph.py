"""Calls captured in a HIP graph and replayed (torch.cuda.CUDAGraph over the library's
stream): the allocation-free decode, which exists for callers that capture their decode
step, and the FP8 prefill into a caller's output. Each replay runs after eager work of the
program's own (clearing the outputs, an eager call of the workspace decode) and a
synchronisation, and must give the eager call's outputs bit for bit."""

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from tests.paths import to_dev
from workloads import custom, generate, page_table, scatter_pages

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _case(*a):
    print("case:", *a, flush=True)


def _decode_inputs(kv_lens, P, Hq, Hkv, D, block, seed):
    B = len(kv_lens)
    table, num_pages = page_table(kv_lens, P, seed)
    rng = np.random.default_rng([980, seed])
    k = rng.standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    v = rng.standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    for i, n in enumerate(kv_lens):
        _, kk, vv = generate(custom(1, Hkv, Hkv, n, D, D, wid=981 + i), seed=seed)
        scatter_pages(k, table[i], kk[0])
        scatter_pages(v, table[i], vv[0])
    q, _, _ = generate(custom(1, B, B, Hq, D, D, wid=990), seed=seed)
    qc, qs = zy.quantize_fp8(to_dev(q[0]).reshape(B, Hkv, Hq // Hkv, D), block)
    kc, ks = zy.quantize_fp8(to_dev(k), block)
    vc, vs = zy.quantize_fp8(to_dev(v), block)
    return (qc.reshape(B, Hq, D), kc, vc, qs, ks, vs, torch.from_numpy(np.array(kv_lens, dtype=np.int32)).cuda(),
            torch.from_numpy(table).cuda())


def _capture(fn):
    """fn captured on a side stream (after one warm call there), as torch's graph API asks."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("lean", [False, True])
def test_noalloc_decode_replays_bitwise(lean):
    kv_lens, P, Hq, Hkv, D, block, split = [1, 300, 2048, 1500], 128, 8, 2, 128, 64, 128
    _case("graph decode", kv_lens, "lean" if lean else "exact")
    qc, kc, vc, qs, ks, vs, kvl, bt = _decode_inputs(kv_lens, P, Hq, Hkv, D, block, seed=5)
    B, mx = len(kv_lens), max(kv_lens)
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def call():
        zy.attn_decode_fp8_paged_noalloc(qc, kc, vc, qs, ks, vs, block, kvl, bt, mx, o, lse, split_keys=split,
                                         lean=lean)

    call()
    torch.cuda.synchronize()
    o_eager, lse_eager = o.clone(), lse.clone()
    g = _capture(call)
    for r in range(REPLAYS):
        o.fill_(0)
        lse.fill_(0)
        o_ws, l_ws = zy.attn_decode_fp8_paged(qc, kc, vc, qs, ks, vs, block, kvl, bt, mx, split_keys=split,
                                              return_lse=True, lean=lean)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {r}", flush=True)
        assert torch.equal(o, o_eager) and torch.equal(lse, lse_eager), f"replay {r}"
        assert torch.equal(o_ws, o_eager) and torch.equal(l_ws, lse_eager)


def test_fp8_prefill_replays_bitwise():
    B, Hq, Hkv, S, D, block = 1, 4, 2, 700, 128, 128
    _case("graph prefill", B, Hq, Hkv, S, D)
    q, k, v = generate(custom(B, Hq, Hkv, S, D, D, wid=995), seed=6)
    (qc, qs), (kc, ks), (vc, vs) = (zy.quantize_fp8(to_dev(x), block) for x in (q, k, v))
    tau = 1.0 / np.sqrt(D)
    o = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device="cuda")

    def call():
        zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, block, tau, o=o)

    call()
    torch.cuda.synchronize()
    o_eager = o.clone()
    g = _capture(call)
    for r in range(REPLAYS):
        o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {r}", flush=True)
        assert torch.equal(o, o_eager), f"replay {r}"
