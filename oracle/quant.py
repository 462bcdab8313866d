"""Input quantization to e4m3 with per-block scales, and the Hadamard rotation.

"ZYFA: Fast and Accurate FP8 Attention on AMD MI355X", section "FP8 Error in
Full-Model Inference" and footnote 2: Q, K and V are quantized to e4m3 before
attention, Q in a pass of its own (with the rotation fused in) and K, V as they
are written to the KV cache; an optional Hadamard rotation of Q and K over the
head dimension leaves Q K^T unchanged and spreads outlier channels.

The pages do not give the scale granularity or formula. The readings used here:

* one float32 scale per (batch, head, block of ``block`` consecutive tokens),
  shared by all head-dim channels; the last block may be shorter;
* amax = max |x| over the block; s = fl32(amax / 448), or s = 1 when
  amax == 0 (the zero guard of the FP8 GEMM on CDNA4 blog, section 2.2);
* code = e4m3(fl32(x / s)): a correctly rounded float32 division, then
  round-to-nearest-even to e4m3 with saturation (blog section 2.3).

The dequantized value of an element is decode(code) * s, exact in float64.
"""

import numpy as np

from .fp8 import E4M3_MAX, e4m3_decode, e4m3_encode


def quantize_blocks(x, block):
    """Quantize float32 ``x`` of shape [B, H, S, D] to e4m3 codes [B, H, S, D]
    (uint8) and float32 scales [B, H, ceil(S / block)]."""
    x = np.asarray(x, dtype=np.float32)
    B, H, S, D = x.shape
    nb = (S + block - 1) // block
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for j in range(nb):
        blk = x[:, :, j * block:(j + 1) * block, :]
        amax = np.abs(blk).max(axis=(2, 3))  # exact: a max of float32 magnitudes
        s = amax / np.float32(E4M3_MAX)  # float32 / float32 -> correctly rounded float32
        s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
        y = blk / s[:, :, None, None]  # correctly rounded float32 division
        codes[:, :, j * block:(j + 1) * block, :] = e4m3_encode(y)
        scales[:, :, j] = s
    return codes, scales


def dequantize_blocks(codes, scales, block):
    """Float64 values decode(code) * scale for codes [B, H, S, D] and scales [B, H, nb]."""
    codes = np.asarray(codes)
    S = codes.shape[2]
    per_token = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :S]
    return e4m3_decode(codes) * per_token[..., None]


def hadamard_matrix(n):
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1, unnormalized:
    H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_rotate(x):
    """Rotate the last axis of ``x`` by the orthonormal Hadamard matrix H_n / sqrt(n),
    in float64: y = x @ (H_n / sqrt(n)). H_n is symmetric, so this is also H x."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    return x @ (hadamard_matrix(n) / np.sqrt(n))
