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
