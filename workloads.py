"""Seeded synthetic inputs for causal prefill attention.

The one module that the GPU path's tests and benchmark share with the oracle's
tests. It draws random numbers and nothing else: no quantization, rotation or
attention arithmetic lives here.

Workloads (named by shape; the first four stand in for the Gaussian kernel
benchmarks of "ZYFA: Fast and Accurate FP8 Attention on AMD MI355X", section
"Throughput on Gaussian Inputs"; the last stands in for its captured
post-RoPE activations, section "Throughput on Captured Activations at Sustained
Clocks", which are not available here):

* ``tiny``   B=1, Hq=Hkv=1, S=128, D=128, Gaussian, FP8 scale block 64.
* ``mha4k``  B=1, Hq=Hkv=32, S=4096, D=128, Gaussian, scale block 128.
* ``gqa32k`` B=1, Hq=32, Hkv=8, S=32768, D=128, Gaussian, scale block 128.
* ``mla32k`` B=1, Hq=Hkv=16, S=32768, Dqk=192, Dv=128, Gaussian, block 128.
* ``act16k`` B=1, Hq=32, Hkv=8, S=16384, D=128, block 128: Q, K ~ N(0, 1)
  with the same 4 of 128 channels scaled by 15 in Q and K, K shifted by a
  per-(KV head, channel) offset ~ N(0, variance 2), V ~ N(0, 1).

Streams: ``numpy.random.default_rng([workload_id, tensor_id, seed])`` with
tensor ids Q=0, K=1, V=2, outlier channels=3, K offset=4.
"""

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    S: int
    Dqk: int
    Dv: int
    scale_block: int
    dist: str = "gaussian"

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.Dqk)

    @property
    def flops(self) -> float:
        """Causal attention FLOPs, FlashAttention convention: 2 (Dqk + Dv) S^2 / 2 per (b, query head)."""
        return 2.0 * (self.Dqk + self.Dv) * self.S * self.S / 2.0 * self.B * self.Hq


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 1, 1, 128, 128, 128, 64),
    "mha4k": Workload("mha4k", 1, 1, 32, 32, 4096, 128, 128, 128),
    "gqa32k": Workload("gqa32k", 2, 1, 32, 8, 32768, 128, 128, 128),
    "mla32k": Workload("mla32k", 3, 1, 16, 16, 32768, 192, 128, 128),
    "act16k": Workload("act16k", 4, 1, 32, 8, 16384, 128, 128, 128, "activation"),
}


def custom(B, Hq, Hkv, S, Dqk=128, Dv=128, scale_block=64, dist="gaussian", wid=100):
    """A workload of any shape (used for small parity and edge cases)."""
    return Workload(f"custom_{B}x{Hq}x{Hkv}x{S}x{Dqk}x{Dv}", wid, B, Hq, Hkv, S, Dqk, Dv, scale_block, dist)


def _rng(w: Workload, tensor_id: int, seed: int):
    return np.random.default_rng([w.wid, tensor_id, seed])


# the "rising" distribution: logit growth per 64 keys (base 2) and the query's weight on
# the shared direction
RISE_BINADES = 5.0
RISE_A = 8.0


def generate(w: Workload, seed: int = 0):
    """Float32 Q [B, Hq, S, Dqk], K [B, Hkv, S, Dqk], V [B, Hkv, S, Dv]."""
    q = _rng(w, 0, seed).standard_normal((w.B, w.Hq, w.S, w.Dqk), dtype=np.float32)
    k = _rng(w, 1, seed).standard_normal((w.B, w.Hkv, w.S, w.Dqk), dtype=np.float32)
    v = _rng(w, 2, seed).standard_normal((w.B, w.Hkv, w.S, w.Dv), dtype=np.float32)
    if w.dist == "activation":
        channels = _rng(w, 3, seed).choice(w.Dqk, size=4, replace=False)
        q[..., channels] *= np.float32(15.0)
        k[..., channels] *= np.float32(15.0)
        offset = _rng(w, 4, seed).normal(0.0, math.sqrt(2.0), size=(w.B, w.Hkv, 1, w.Dqk)).astype(np.float32)
        k += offset
    elif w.dist == "rising":
        # Scores that climb along the key axis: q_i . k_j carries a term A * RISE_B * j
        # along one random unit direction per KV head, so that with the softmax scale
        # 1/sqrt(Dqk) the base-2 logits gain about RISE_BINADES per 64 keys and every
        # row's running maximum keeps growing (stress input for the online softmax).
        tau_log2e = math.log2(math.e) / math.sqrt(w.Dqk)
        slope = RISE_BINADES / (64.0 * tau_log2e * RISE_A)
        u = _rng(w, 3, seed).standard_normal((w.B, w.Hkv, 1, w.Dqk))
        u /= np.linalg.norm(u, axis=-1, keepdims=True)
        q += (RISE_A * np.repeat(u, w.Hq // w.Hkv, axis=1)).astype(np.float32)
        k += (slope * np.arange(w.S, dtype=np.float64)[None, None, :, None] * u).astype(np.float32)
    elif w.dist != "gaussian":
        raise ValueError(f"unknown distribution {w.dist}")
    return q, k, v


def sample_rows(S: int, n: int, seed: int = 0):
    """Sorted query rows for sampled checks: the first and last rows, plus a seeded
    spread over the whole sequence."""
    rng = np.random.default_rng([999, S, seed])
    fixed = [0, 1, S // 2, S - 1]
    extra = rng.choice(S, size=max(0, min(n, S) - len(fixed)), replace=False)
    return np.unique(np.concatenate([np.array(fixed), extra]).clip(0, S - 1))


def page_table(kv_lens, page_size: int, seed: int = 0, spare: int = 3):
    """A shuffled layout of a paged key/value cache: sequence i needs
    ceil(kv_lens[i] / page_size) pages, taken in a seeded random order from a cache of
    that many pages plus `spare` unused ones. Returns (block_table int32 [n, max_pages],
    num_pages); table entries past a sequence's pages hold -1."""
    need = [-(-int(n) // page_size) for n in kv_lens]
    num_pages = sum(need) + spare
    perm = np.random.default_rng([777, page_size, seed]).permutation(num_pages)
    table = np.full((len(need), max(1, max(need))), -1, dtype=np.int32)
    at = 0
    for i, m in enumerate(need):
        table[i, :m] = perm[at:at + m]
        at += m
    return table, num_pages


def scatter_pages(cache, table_row, x):
    """Write x [H, n, D] (one sequence's tokens) into cache [pages, H, P, D] at the pages
    table_row lists, in order (data placement only)."""
    P = cache.shape[2]
    for j in range(-(-x.shape[1] // P)):
        part = x[:, j * P:(j + 1) * P]
        cache[int(table_row[j]), :, :part.shape[1]] = part
