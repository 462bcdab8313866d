"""Pins for the oracle's windowed attention (a chunk of query rows against a window of
keys) and its merge of partial results.

Neither function is checked against a retyping of itself. They are pinned by: reduction
to the pinned causal attention (the whole window and offset 0; a chunk of rows against
its causal prefix), the identity that splitting the keys into windows and merging the
parts gives one pass over all keys (a mistake in either function, such as an off-by-one
window edge or a wrong merge weight, breaks it), exact zeros and -inf for rows that see no
key, brute force in 50-digit arithmetic, torch's float64 scaled_dot_product_attention with
an explicit mask (a library routine), and invariants of the merge (order of the parts,
grouping, a repeated part, parts that saw nothing, log-sum-exp values far outside exp's
range).
"""

import math

import mpmath
import numpy as np
import pytest
import torch

from oracle import causal_attention, merge_partials, window_attention


def _qkv(B, Hq, Hkv, Sq, Skv, Dqk, Dv, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Sq, Dqk)) * scale
    k = rng.standard_normal((B, Hkv, Skv, Dqk)) * scale
    v = rng.standard_normal((B, Hkv, Skv, Dv))
    return q, k, v


def test_whole_window_equals_causal_attention():
    q, k, v = _qkv(2, 4, 2, 77, 77, 32, 16, seed=1)
    o1, l1 = causal_attention(q, k, v, 0.3)
    o2, l2 = window_attention(q, k, v, 0.3)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("a,b", [(0, 40), (40, 100), (63, 64), (99, 130)])
def test_chunk_of_rows_equals_causal_rows(a, b):
    q, k, v = _qkv(1, 2, 1, 130, 130, 16, 8, seed=2, scale=1.4)
    o_full, l_full = causal_attention(q, k, v, 0.5)
    # rows a..b-1 as a chunk at offset a, against the keys of positions 0..b-1
    o, l = window_attention(q[:, :, a:b], k[:, :, :b], v[:, :, :b], 0.5, q_offset=a)
    assert np.allclose(o, o_full[:, :, a:b], rtol=0, atol=1e-13)
    assert np.allclose(l, l_full[:, :, a:b], rtol=0, atol=1e-13)
    # longer key tensors do not change anything: keys past a row's position stay masked
    o2, l2 = window_attention(q[:, :, a:b], k, v, 0.5, q_offset=a)
    assert np.allclose(o2, o, rtol=0, atol=1e-13) and np.allclose(l2, l, rtol=0, atol=1e-13)


@pytest.mark.parametrize("cuts,shape", [
    ([64], (1, 2, 2, 200, 32, 32)),
    ([64, 192], (2, 4, 2, 300, 128, 128)),
    ([128, 129, 256], (1, 2, 1, 260, 192, 128)),
])
def test_split_windows_merge_to_one_pass(cuts, shape):
    B, Hq, Hkv, S, Dqk, Dv = shape
    q, k, v = _qkv(B, Hq, Hkv, S, S, Dqk, Dv, seed=3, scale=1.2)
    tau = 1 / math.sqrt(Dqk)
    edges = [0] + cuts + [S]
    parts = [window_attention(q, k, v, tau, k_begin=lo, k_end=hi) for lo, hi in zip(edges[:-1], edges[1:])]
    o, l = merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    o_ref, l_ref = causal_attention(q, k, v, tau)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.allclose(l, l_ref, rtol=0, atol=1e-12)
    # the parts are not trivially equal to the whole: a later window changes late rows
    assert not np.allclose(parts[0][0][:, :, -1], o_ref[:, :, -1], atol=1e-3)


def test_rows_without_keys_are_zero_and_minus_inf():
    q, k, v = _qkv(1, 2, 2, 50, 200, 16, 16, seed=4)
    # rows at positions 10..59 against keys [40, 120): rows at positions < 40 see nothing
    o, l = window_attention(q, k, v, 0.4, q_offset=10, k_begin=40, k_end=120)
    empty = np.arange(50) + 10 < 40
    assert np.all(o[:, :, empty] == 0.0) and np.all(l[:, :, empty] == -np.inf)
    assert np.all(np.isfinite(l[:, :, ~empty]))
    # position 40 sees exactly key 40
    assert np.array_equal(o[:, :, 30], v[:, :, 40])


@pytest.mark.parametrize("q_offset,k_begin,k_end", [(3, 2, 9), (0, 4, 12), (6, 0, 5)])
def test_window_brute_force_mpmath(q_offset, k_begin, k_end):
    mpmath.mp.dps = 50
    Sq, Skv, D, Dv = 7, 12, 4, 3
    q, k, v = _qkv(1, 1, 1, Sq, Skv, D, Dv, seed=5 + q_offset, scale=1.6)
    tau = 0.7
    o, lse = window_attention(q, k, v, tau, q_offset=q_offset, k_begin=k_begin, k_end=k_end)
    for i in range(Sq):
        keys = [j for j in range(Skv) if k_begin <= j < k_end and j <= q_offset + i]
        if not keys:
            assert np.all(o[0, 0, i] == 0) and lse[0, 0, i] == -np.inf
            continue
        s = [mpmath.mpf(tau) * mpmath.fsum(mpmath.mpf(q[0, 0, i, d]) * mpmath.mpf(k[0, 0, j, d]) for d in range(D))
             for j in keys]
        w = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(w)
        for c in range(Dv):
            ref = mpmath.fsum(wj * mpmath.mpf(v[0, 0, j, c]) for wj, j in zip(w, keys)) / z
            assert abs(float(ref) - o[0, 0, i, c]) <= 1e-14 * max(1.0, abs(float(ref)))
        assert abs(float(mpmath.log(z)) - lse[0, 0, i]) <= 1e-13 * max(1.0, abs(float(mpmath.log(z))))


def test_window_against_torch_sdpa_with_mask():
    B, Hq, Hkv, Sq, Skv, Dqk, Dv = 1, 4, 2, 90, 300, 128, 128
    q, k, v = _qkv(B, Hq, Hkv, Sq, Skv, Dqk, Dv, seed=6, scale=1.3)
    tau = 1 / math.sqrt(Dqk)
    q_offset, k_begin, k_end = 150, 64, 220
    o, lse = window_attention(q, k, v, tau, q_offset=q_offset, k_begin=k_begin, k_end=k_end)
    j = torch.arange(Skv)
    i = torch.arange(Sq)[:, None] + q_offset
    mask = (j >= k_begin) & (j < k_end) & (j <= i)
    assert bool(mask.any(dim=1).all())  # every row sees a key here
    g = Hq // Hkv
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(np.repeat(k, g, axis=1)).contiguous()
    vt = torch.from_numpy(np.repeat(v, g, axis=1)).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=tau).numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-12)
    scores = ((qt @ kt.transpose(-1, -2)) * tau).masked_fill(~mask, float("-inf"))
    assert np.allclose(lse, torch.logsumexp(scores, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_merge_invariants():
    rng = np.random.default_rng(7)
    P, R, Dv = 4, 30, 8
    o = rng.standard_normal((P, R, Dv))
    l = rng.standard_normal((P, R)) * 5
    l[1, :10] = -np.inf  # part 1 saw no key of rows 0..9
    l[:, 29] = -np.inf   # no part saw row 29
    m, lm = merge_partials(o, l)
    # a single part is returned unchanged (row 29, which it did not see, becomes 0)
    m1, l1 = merge_partials(o[:1], l[:1])
    assert np.array_equal(m1[:29], o[0, :29]) and np.array_equal(l1, l[0]) and np.all(m1[29] == 0)
    # order of the parts and grouping of the merges do not matter
    mp_, lp_ = merge_partials(o[::-1], l[::-1])
    assert np.allclose(mp_, m, rtol=0, atol=1e-13) and np.allclose(lp_, lm, rtol=0, atol=1e-13)
    ma, la = merge_partials(o[:2], l[:2])
    mb, lb = merge_partials(o[2:], l[2:])
    mg, lg = merge_partials(np.stack([ma, mb]), np.stack([la, lb]))
    assert np.allclose(mg[:29], m[:29], rtol=0, atol=1e-12) and np.allclose(lg, lm, rtol=0, atol=1e-12)
    # a part that saw nothing contributes nothing
    m_wo, l_wo = merge_partials(o[[0, 2, 3]], l[[0, 2, 3]])
    assert np.allclose(m_wo[:10], m[:10], rtol=0, atol=1e-13) and np.allclose(l_wo[:10], lm[:10], rtol=0, atol=1e-13)
    # a row no part saw
    assert np.all(m[29] == 0) and lm[29] == -np.inf
    # the same part twice: the output is unchanged and the log-sum-exp grows by ln 2
    m2, l2 = merge_partials(np.stack([o[0], o[0]]), np.stack([l[0], l[0]]))
    assert np.allclose(m2[:29], o[0, :29], rtol=0, atol=1e-13)
    assert np.allclose(l2[:29], l[0, :29] + math.log(2), rtol=0, atol=1e-13)
    # log-sum-exp values far outside exp's range
    mh, lh = merge_partials(np.stack([o[0], o[1]]), np.stack([np.full(R, 2000.0), np.full(R, 2000.0)]))
    assert np.allclose(mh, (o[0] + o[1]) / 2, rtol=0, atol=1e-13) and np.allclose(lh, 2000 + math.log(2))


def test_varlen_is_each_sequence_on_its_own():
    # three sequences of different lengths packed with gaps between them: each equals the
    # causal oracle on its own slice (mpmath-pinned), gaps are 0 / -inf, and no sequence
    # sees another's keys (changing one sequence's K/V leaves the others bit for bit)
    from oracle import varlen_attention
    rng = np.random.default_rng(11)
    Hq, Hkv, T, D = 4, 2, 400, 32
    q = rng.standard_normal((Hq, T, D))
    k = rng.standard_normal((Hkv, T, D))
    v = rng.standard_normal((Hkv, T, D))
    cu = [0, 64, 64, 192, 320, 390]  # an empty sequence, and tokens 390..399 outside all
    o, lse = varlen_attention(q, k, v, 0.3, cu)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        if s1 > s0:
            ro, rl = causal_attention(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1], 0.3)
            assert np.array_equal(o[:, s0:s1], ro[0]) and np.array_equal(lse[:, s0:s1], rl[0])
    assert np.all(o[:, 390:] == 0) and np.all(lse[:, 390:] == -np.inf)
    k2, v2 = k.copy(), v.copy()
    k2[:, 192:320] += 5.0
    v2[:, 192:320] *= -1.0
    o2, _ = varlen_attention(q, k2, v2, 0.3, cu)
    assert np.array_equal(o2[:, :192], o[:, :192]) and np.array_equal(o2[:, 320:], o[:, 320:])
    assert not np.allclose(o2[:, 192:320], o[:, 192:320])
    # a row subset (the matrix products see other shapes: equal up to rounding order)
    rows = np.array([0, 63, 64, 250, 389, 395])
    os_, ls_ = varlen_attention(q, k, v, 0.3, cu, rows=rows)
    assert np.allclose(os_, o[:, rows], rtol=0, atol=1e-13)
    assert np.array_equal(np.isfinite(ls_), np.isfinite(lse[:, rows]))
    fin = np.isfinite(ls_)
    assert np.allclose(ls_[fin], lse[:, rows][fin], rtol=0, atol=1e-13)


def test_paged_attention_is_the_chunk_against_its_gathered_prefix():
    # sequences whose keys/values live in shuffled pages of a cache: each chunk equals the
    # causal oracle's last rows on the contiguous sequence (pinned above), whatever the page
    # order; rows outside every chunk are 0 / -inf
    from oracle import paged_attention
    rng = np.random.default_rng(12)
    Hq, Hkv, D, P = 4, 2, 16, 64
    lens = [200, 64, 130]        # tokens per sequence, cached
    chunk = [72, 64, 1]          # new tokens per sequence (its last ones)
    n_pages = sum(-(-n // P) for n in lens) + 3
    perm = rng.permutation(n_pages)
    seqs, tables, used = [], [], 0
    k_cache = rng.standard_normal((n_pages, Hkv, P, D))
    v_cache = rng.standard_normal((n_pages, Hkv, P, D))
    for n in lens:
        npg = -(-n // P)
        pages = perm[used:used + npg]
        used += npg
        tables.append(np.concatenate([pages, np.zeros(8 - npg, dtype=np.int64)]))
        seqs.append((np.concatenate([k_cache[p] for p in pages], axis=1)[:, :n],
                     np.concatenate([v_cache[p] for p in pages], axis=1)[:, :n]))
    cu = np.concatenate([[0], np.cumsum(chunk)])
    T = cu[-1] + 5
    full_q = [rng.standard_normal((Hq, n, D)) for n in lens]
    q = np.zeros((Hq, T, D))
    for i, (s0, s1) in enumerate(zip(cu[:-1], cu[1:])):
        q[:, s0:s1] = full_q[i][:, lens[i] - chunk[i]:]
    o, lse = paged_attention(q, k_cache, v_cache, 0.25, cu, lens, np.stack(tables))
    for i, (s0, s1) in enumerate(zip(cu[:-1], cu[1:])):
        k, v = seqs[i]
        ro, rl = causal_attention(full_q[i][None], k[None], v[None], 0.25)
        assert np.allclose(o[:, s0:s1], ro[0, :, lens[i] - chunk[i]:], rtol=0, atol=1e-12)
        assert np.allclose(lse[:, s0:s1], rl[0, :, lens[i] - chunk[i]:], rtol=0, atol=1e-12)
    assert np.all(o[:, cu[-1]:] == 0) and np.all(lse[:, cu[-1]:] == -np.inf)
