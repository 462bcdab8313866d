"""Pins for the oracle's fp64 causal attention.

The oracle is the plain definition of causal softmax attention. It is pinned
here, without re-deriving it from itself, by: closed forms (row 0 returns v0;
equal scores return the prefix mean of V; constant V returns that constant; a
dominant score returns its key's value), invariants (probability rows sum to
one; a common shift of all keys; GQA equals MHA with repeated K/V; an
orthonormal Hadamard rotation of Q and K; affine maps of V), brute force in
50-digit arithmetic (mpmath) on tiny inputs, and torch's float64
scaled_dot_product_attention with is_causal=True (a library routine).
"""

import math

import mpmath
import numpy as np
import pytest
import torch

from oracle import causal_attention, causal_probs, hadamard_rotate


def _qkv(B, Hq, Hkv, S, Dqk, Dv, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, Dqk)) * scale
    k = rng.standard_normal((B, Hkv, S, Dqk)) * scale
    v = rng.standard_normal((B, Hkv, S, Dv))
    return q, k, v


def test_probability_rows_sum_to_one_and_are_causal():
    q, k, _ = _qkv(1, 1, 1, 50, 16, 16, seed=1, scale=2.0)
    p = causal_probs(q[0, 0], k[0, 0], 0.3)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[np.triu_indices(50, 1)] == 0)
    assert np.all(p[np.tril_indices(50)] > 0)


def _torch_probs(q, k, scale):
    """Causal softmax by torch's float64 softmax over masked scores (a library routine)."""
    s = torch.from_numpy(q) @ torch.from_numpy(k).T * scale
    S = s.shape[0]
    s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    return torch.softmax(s, dim=-1).numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("scale", [0.3, 1 / math.sqrt(64)])
def test_probabilities_match_library_softmax_and_attention(scale):
    # "Error of a Single Attention Call" (ZYFA): P is the causal softmax of scale * Q K^T.
    # Pinned by torch's softmax of the masked scores, and by P V = the oracle's attention
    # output (itself pinned by SDPA and brute force below). A dropped or doubled scale
    # changes P by far more than the tolerance.
    q, k, v = _qkv(1, 1, 1, 70, 64, 32, seed=11, scale=1.3)
    q, k, v = q[0, 0], k[0, 0], v[0, 0]
    p = causal_probs(q, k, scale)
    pt, lse_t = _torch_probs(q, k, scale)
    assert np.allclose(p, pt, rtol=1e-12, atol=1e-15)
    o, lse = causal_attention(q[None, None], k[None, None], v[None, None], scale)
    assert np.allclose(p @ v, o[0, 0], rtol=0, atol=1e-13)
    assert np.allclose(lse[0, 0], lse_t, rtol=0, atol=1e-12)
    # log P_ij + LSE_i is the scaled score of every visible pair
    i, j = np.tril_indices(70)
    assert np.allclose(np.log(p[i, j]) + lse[0, 0][i], scale * np.sum(q[i] * k[j], axis=1), rtol=0, atol=1e-11)
    for wrong in (2 * scale, 1.0):
        assert not np.allclose(causal_probs(q, k, wrong), pt, rtol=1e-6, atol=1e-9)


def test_row0_returns_v0():
    q, k, v = _qkv(2, 4, 2, 33, 128, 128, seed=2)
    o, lse = causal_attention(q, k, v, 1 / math.sqrt(128))
    for h in range(4):
        assert np.array_equal(o[:, h, 0], v[:, h // 2, 0])
    assert np.allclose(lse[:, :, 0], np.einsum("bhd,bhd->bh", q[:, :, 0], np.repeat(k, 2, axis=1)[:, :, 0]) / math.sqrt(128))


def test_equal_scores_give_prefix_mean():
    _, k, v = _qkv(1, 2, 2, 40, 64, 32, seed=3)
    q = np.zeros((1, 2, 40, 64))
    o, lse = causal_attention(q, k, v, 0.125)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, 41)[None, None, :, None]
    assert np.allclose(o, prefix_mean, rtol=0, atol=1e-13)
    assert np.allclose(lse, np.log(np.arange(1, 41))[None, None, :], rtol=0, atol=1e-13)


def test_constant_v_and_affine_v():
    q, k, v = _qkv(1, 2, 1, 30, 32, 16, seed=4, scale=1.5)
    ones = np.full_like(v, 2.5)
    o, _ = causal_attention(q, k, ones, 0.2)
    assert np.allclose(o, 2.5, rtol=0, atol=1e-13)
    o1, _ = causal_attention(q, k, v, 0.2)
    o2, _ = causal_attention(q, k, 3.0 * v - 7.0, 0.2)
    assert np.allclose(o2, 3.0 * o1 - 7.0, rtol=0, atol=1e-12)


def test_dominant_score_selects_its_value():
    q, k, v = _qkv(1, 1, 1, 20, 8, 8, seed=5, scale=0.1)
    q[0, 0, 15] = 0.0
    q[0, 0, 15, 0] = 1.0
    k[0, 0, 9, 0] = 1000.0  # s(15, 9) = 1000 * scale, the rest are O(0.1)
    o, _ = causal_attention(q, k, v, 1.0)
    assert np.allclose(o[0, 0, 15], v[0, 0, 9], rtol=0, atol=1e-12)
    # rows before 9 cannot see key 9
    assert not np.allclose(o[0, 0, 8], v[0, 0, 9], atol=1e-3)


def test_common_key_shift_is_invariant():
    q, k, v = _qkv(1, 2, 2, 25, 16, 16, seed=6)
    u = np.random.default_rng(60).standard_normal(16) * 3
    o1, _ = causal_attention(q, k, v, 0.5)
    o2, _ = causal_attention(q, k + u, v, 0.5)
    assert np.allclose(o1, o2, rtol=0, atol=1e-11)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = _qkv(2, 8, 2, 24, 32, 16, seed=7)
    o_gqa, l_gqa = causal_attention(q, k, v, 0.3)
    o_mha, l_mha = causal_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.3)
    assert np.array_equal(o_gqa, o_mha) and np.array_equal(l_gqa, l_mha)
    # query head h uses key/value head h // 4: head 5 must differ from a run with kv head 0
    o_wrong, _ = causal_attention(q[:, 5:6], k[:, 0:1], v[:, 0:1], 0.3)
    assert not np.allclose(o_wrong[:, 0], o_gqa[:, 5])


def test_hadamard_rotation_of_q_and_k_is_invariant():
    q, k, v = _qkv(1, 2, 1, 32, 128, 128, seed=8)
    o1, l1 = causal_attention(q, k, v, 1 / math.sqrt(128))
    o2, l2 = causal_attention(hadamard_rotate(q), hadamard_rotate(k), v, 1 / math.sqrt(128))
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)
    assert np.allclose(l1, l2, rtol=0, atol=1e-12)


def test_row_subset_matches_full():
    q, k, v = _qkv(1, 3, 3, 300, 64, 64, seed=9)
    rows = np.array([0, 5, 64, 199, 200, 299])
    o_full, l_full = causal_attention(q, k, v, 0.2, row_chunk=37)
    o_sub, l_sub = causal_attention(q, k, v, 0.2, rows=rows, row_chunk=4)
    assert np.allclose(o_full[:, :, rows], o_sub, rtol=0, atol=1e-13)
    assert np.allclose(l_full[:, :, rows], l_sub, rtol=0, atol=1e-13)


@pytest.mark.parametrize("S", [1, 2, 7, 16])
def test_brute_force_mpmath(S):
    mpmath.mp.dps = 50
    D, Dv = 4, 3
    q, k, v = _qkv(1, 1, 1, S, D, Dv, seed=10 + S, scale=1.7)
    tau = 0.61
    o, lse = causal_attention(q, k, v, tau)
    for i in range(S):
        s = [mpmath.mpf(tau) * mpmath.fsum(mpmath.mpf(q[0, 0, i, d]) * mpmath.mpf(k[0, 0, j, d]) for d in range(D))
             for j in range(i + 1)]
        w = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(w)
        for c in range(Dv):
            ref = mpmath.fsum(w[j] * mpmath.mpf(v[0, 0, j, c]) for j in range(i + 1)) / z
            assert abs(float(ref) - o[0, 0, i, c]) <= 1e-14 * max(1.0, abs(float(ref)))
        assert abs(float(mpmath.log(z)) - lse[0, 0, i]) <= 1e-13 * max(1.0, abs(float(mpmath.log(z))))


@pytest.mark.parametrize("shape", [(1, 4, 4, 70, 128, 128), (2, 8, 2, 45, 192, 128)])
def test_against_torch_sdpa_float64(shape):
    B, Hq, Hkv, S, Dqk, Dv = shape
    q, k, v = _qkv(B, Hq, Hkv, S, Dqk, Dv, seed=11, scale=1.3)
    tau = 1 / math.sqrt(Dqk)
    o, lse = causal_attention(q, k, v, tau)
    g = Hq // Hkv
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(np.repeat(k, g, axis=1)).contiguous()
    vt = torch.from_numpy(np.repeat(v, g, axis=1)).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=tau).numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-12)
    scores = (qt @ kt.transpose(-1, -2)) * tau
    scores = scores.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    assert np.allclose(lse, torch.logsumexp(scores, dim=-1).numpy(), rtol=0, atol=1e-12)
