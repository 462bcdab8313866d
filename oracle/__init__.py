"""FP64 CPU oracle for causal prefill attention in FP8 (OCP e4m3) and BF16.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
reference that the GPU path is judged against. Only the test suite, the smoke
check of the package entry point and the CPU-baseline leg of the benchmark may
import it; the GPU library and its Python binding never do, and the two share
no code (inputs come from the seeded generators in ``workloads``, which hold
none of the method's arithmetic).

Sources (cited by page title and section):

* "ZYFA: Fast and Accurate FP8 Attention on AMD MI355X" (hot.atechcom.net; its
  Russian translation on dev48.org is used to repair extraction damage).
  - Introduction: the kernel is causal forward attention, softmax(Q K^T *
    scale + causal mask) V, at head dim 128 and the MLA shape (192 / 128).
  - "Error of a Single Attention Call": a kernel is judged against fp64
    attention evaluated on the same quantized inputs.
  - "FP8 Error in Full-Model Inference": Q, K and V are quantized to e4m3;
    an optional Hadamard rotation of Q and K over the head dimension.
  - footnote 7 and "Precision and Underflow of FP8 Probabilities": the e4m3
    code points and thresholds.
  - "Methodology and Limitations": equal query and key lengths.
* Zyphra "Inference Wave 2", section on CSA dual-scope decode: keys split
  into shards, each returning a partial output and its log-sum-exp, merged
  into the result of one pass.
* The FP8 GEMM on CDNA4 practitioner's blog (kwkr.cn), sections 2.1-2.3:
  e4m3 range (max 448), absmax block scaling with a zero guard, and
  round-to-nearest-even.

Modules:

* ``fp8``       - e4m3 (OCP E4M3FN) decode / round-to-nearest-even encode,
                  bfloat16 round-to-nearest-even.
* ``quant``     - per-(batch, head, token-block) absmax quantizer and the
                  Hadamard rotation (Sylvester order 128; order 192 as the
                  Kronecker product of Paley's order-12 matrix and Sylvester's 16).
* ``attention`` - fp64 causal attention with GQA and log-sum-exp, over all
                  rows or a chosen subset of query rows; the same for a chunk of
                  query rows against a window of keys, the merge of partial
                  results over disjoint key sets, batches of sequences of
                  different lengths packed along the token axis, and chunks of new
                  tokens against a paged key/value cache.

Every function here is pinned by tests that do not re-derive it from itself:
printed code points, closed forms, invariants, brute force in 50-digit
arithmetic and library routines (torch float8/bfloat16 casts, SciPy's
Hadamard matrix, torch's float64 scaled_dot_product_attention).
"""

from .fp8 import (E4M3_MAX, e4m3_decode, e4m3_encode, bf16_round, bf16_bits_to_f64,
                  f32_to_bf16_bits)
from .quant import quantize_blocks, dequantize_blocks, hadamard_matrix, hadamard_rotate, paley_hadamard_12
from .attention import (causal_attention, causal_probs, gather_pages, merge_partials, paged_attention,
                        varlen_attention, window_attention)

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "bf16_round", "bf16_bits_to_f64", "f32_to_bf16_bits",
    "quantize_blocks", "dequantize_blocks", "hadamard_matrix", "hadamard_rotate", "paley_hadamard_12",
    "causal_attention", "causal_probs", "window_attention", "merge_partials", "varlen_attention",
    "gather_pages", "paged_attention",
]
