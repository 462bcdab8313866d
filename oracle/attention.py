"""FP64 causal attention: the definition the kernels are judged against.

"ZYFA: Fast and Accurate FP8 Attention on AMD MI355X":

* Introduction: causal forward attention O = softmax(Q K^T * scale + causal
  mask) V, with head dim 128 (query heads may share a key/value head: GQA)
  and the MLA shape, query-key dim 192 and value dim 128 (footnote 4).
* "Methodology and Limitations": queries and keys have equal lengths, so
  query i attends to keys j <= i.
* "Error of a Single Attention Call": the reference is fp64 attention on the
  same (dequantized) inputs the kernel read.

Per batch b and query head h, with key/value head g = h // (Hq / Hkv) (the
grouping reading: consecutive query heads share a key/value head):

    s_ij = scale * sum_d Q[b,h,i,d] K[b,g,j,d]      for j <= i
    m_i  = max_j s_ij
    w_ij = exp(s_ij - m_i)
    O_i  = sum_j w_ij V[b,g,j,:] / sum_j w_ij
    LSE_i = m_i + ln sum_j w_ij

Rows are processed in chunks only to bound memory; each row is computed
independently and exactly as written above.
"""

import numpy as np


def causal_probs(q, k, scale):
    """Attention probabilities of one head: q [S, D], k [S, D] -> P [S, S] (float64),
    P_ij = exp(s_ij - m_i) / sum_j exp(s_ij - m_i) for j <= i and 0 for j > i."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    S = q.shape[0]
    s = scale * (q @ k.T)
    s = np.where(np.tril(np.ones((S, S), dtype=bool)), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return w / w.sum(axis=1, keepdims=True)


def causal_attention(q, k, v, scale, rows=None, row_chunk=256):
    """Causal attention in float64.

    q: [B, Hq, S, Dqk], k: [B, Hkv, S, Dqk], v: [B, Hkv, S, Dv] (any float dtype,
    promoted to float64). ``rows``: None for every query row, or a 1-D array of
    query indices. Returns (o [B, Hq, R, Dv], lse [B, Hq, R]) in float64, R the
    number of rows computed; lse is the natural-log log-sum-exp of the scaled
    scores."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, _ = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    o = np.empty((B, Hq, R, v.shape[3]))
    lse = np.empty((B, Hq, R))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for c0 in range(0, R, row_chunk):
                idx = rows[c0:c0 + row_chunk]
                n = int(idx.max()) + 1  # keys beyond the last row's position are all masked
                s = scale * (q[b, h, idx] @ k[b, g, :n].T)
                s = np.where(np.arange(n)[None, :] <= idx[:, None], s, -np.inf)
                m = s.max(axis=1)
                w = np.exp(s - m[:, None])
                l = w.sum(axis=1)
                o[b, h, c0:c0 + len(idx)] = (w @ v[b, g, :n]) / l[:, None]
                lse[b, h, c0:c0 + len(idx)] = m + np.log(l)
    return o, lse


def window_attention(q, k, v, scale, q_offset=0, k_begin=0, k_end=None, rows=None, row_chunk=256):
    """Causal attention of a chunk of query rows against a window of keys, in float64.

    Zyphra "Inference Wave 2", section on CSA dual-scope decode: the keys of one call may
    be split into shards, each giving a partial output and the log-sum-exp of its scores;
    the ZYFA Introduction fixes the causal rule (a query sees keys up to its own position).

    q: [B, Hq, Sq, Dqk], query row i being the token at sequence position q_offset + i.
    k: [B, Hkv, Skv, Dqk], v: [B, Hkv, Skv, Dv], key j being the token at position j.
    Key j is visible to row i iff k_begin <= j < k_end and j <= q_offset + i (k_end
    defaults to Skv). Over the visible keys, O_i and LSE_i are as in causal_attention; a
    row with no visible key has O_i = 0 and LSE_i = -inf (a part that holds none of the
    row's keys). ``rows``: None for every row, or the row indices to compute."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if k_end is None:
        k_end = Skv
    group = Hq // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    j = np.arange(Skv)
    o = np.zeros((B, Hq, R, v.shape[3]))
    lse = np.full((B, Hq, R), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for c0 in range(0, R, row_chunk):
                idx = rows[c0:c0 + row_chunk]
                visible = (j[None, :] >= k_begin) & (j[None, :] < k_end) & (j[None, :] <= q_offset + idx[:, None])
                seen = visible.any(axis=1)
                if not seen.any():
                    continue
                s = scale * (q[b, h, idx[seen]] @ k[b, g].T)
                s = np.where(visible[seen], s, -np.inf)
                m = s.max(axis=1)
                w = np.exp(s - m[:, None])
                l = w.sum(axis=1)
                out = np.flatnonzero(seen) + c0
                o[b, h, out] = (w @ v[b, g]) / l[:, None]
                lse[b, h, out] = m + np.log(l)
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine partial attention results over disjoint key sets, in float64.

    Zyphra "Inference Wave 2", section on CSA dual-scope decode: partial outputs and their
    log-sum-exp statistics merge into the result of one pass over all keys. With parts p
    of one row: M = max_p LSE_p, w_p = exp(LSE_p - M), O = sum_p w_p O_p / sum_p w_p,
    LSE = M + ln sum_p w_p. A part with LSE_p = -inf holds no key of the row and has weight
    zero; a row that no part saw gets O = 0, LSE = -inf.

    o_parts: [P, ..., Dv]; lse_parts: [P, ...]. Returns (o [..., Dv], lse [...])."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    seen = m > -np.inf
    w = np.where(seen[None], np.exp(lse_parts - np.where(seen, m, 0.0)[None]), 0.0)
    wsum = w.sum(axis=0)
    o = np.zeros(o_parts.shape[1:])
    o[seen] = (np.einsum("p...,p...d->...d", w, o_parts)[seen]) / wsum[seen][:, None]
    lse = np.where(seen, m + np.log(np.where(seen, wsum, 1.0)), -np.inf)
    return o, lse


def varlen_attention(q, k, v, scale, cu_seqlens, rows=None):
    """Causal attention over a batch of sequences of different lengths, packed along the
    token axis, in float64 (the ZYFA page's "Future Work" lists batches of variable length;
    each sequence is the page's causal prefill on its own).

    q: [Hq, T, Dqk], k: [Hkv, T, Dqk], v: [Hkv, T, Dv]; sequence i occupies tokens
    cu_seqlens[i] .. cu_seqlens[i+1] - 1 of every head, and its query rows attend causally
    to its own keys only. Tokens outside every sequence get O = 0 and LSE = -inf.
    ``rows``: None, or packed token indices to compute (returned in that order).
    Returns (o [Hq, R, Dv], lse [Hq, R])."""
    q = np.asarray(q, dtype=np.float64)
    Hq, T, _ = q.shape
    cu = [int(c) for c in cu_seqlens]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((Hq, rows.shape[0], np.asarray(v).shape[2]))
    lse = np.full((Hq, rows.shape[0]), -np.inf)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        sel = np.flatnonzero((rows >= s0) & (rows < s1))
        if s1 <= s0 or sel.size == 0:
            continue
        oi, li = causal_attention(q[None, :, s0:s1], np.asarray(k)[None, :, s0:s1], np.asarray(v)[None, :, s0:s1],
                                  scale, rows=rows[sel] - s0)
        o[:, sel] = oi[0]
        lse[:, sel] = li[0]
    return o, lse


def gather_pages(cache, block_table, n_tokens):
    """The first n_tokens tokens of one sequence from a paged cache, in float64: cache
    [pages, H, P, D] holds P tokens of every head per page; block_table lists the
    sequence's pages in order (logical page j of the sequence is cache[block_table[j]]).
    Returns [H, n_tokens, D]."""
    cache = np.asarray(cache)
    P = cache.shape[2]
    n_pages = -(-n_tokens // P)
    pages = [cache[int(block_table[j])] for j in range(n_pages)]  # each [H, P, D]
    return np.concatenate(pages, axis=1)[:, :n_tokens].astype(np.float64)


def paged_attention(q, k_cache, v_cache, scale, cu_seqlens, kv_lens, block_table):
    """Attention of chunks of new tokens against their sequences' cached keys, in float64
    (prefill into a paged key/value cache; the ZYFA page's "Future Work" lists paged KV
    caches). q: [Hq, T, Dqk], sequence i's new tokens being rows cu_seqlens[i] ..
    cu_seqlens[i+1] - 1; they are the last L_i of the sequence's kv_lens[i] tokens, whose
    keys and values sit in the pages block_table[i] of k_cache / v_cache
    ([pages, Hkv, P, D]). Row r of the chunk is at position kv_lens[i] - L_i + r and sees
    the sequence's keys up to it (window_attention). Rows outside every chunk get O = 0,
    LSE = -inf. Returns (o [Hq, T, Dv], lse [Hq, T])."""
    q = np.asarray(q, dtype=np.float64)
    Hq, T, _ = q.shape
    cu = [int(c) for c in cu_seqlens]
    o = np.zeros((Hq, T, np.asarray(v_cache).shape[3]))
    lse = np.full((Hq, T), -np.inf)
    for i, (s0, s1) in enumerate(zip(cu[:-1], cu[1:])):
        if s1 <= s0:
            continue
        n = int(kv_lens[i])
        k = gather_pages(k_cache, block_table[i], n)
        v = gather_pages(v_cache, block_table[i], n)
        oi, li = window_attention(q[None, :, s0:s1], k[None], v[None], scale, q_offset=n - (s1 - s0))
        o[:, s0:s1] = oi[0]
        lse[:, s0:s1] = li[0]
    return o, lse
