"""Input quantization to e4m3 with per-block scales, and the Hadamard rotation.

"ZYFA: Fast and Accurate FP8 Attention on AMD MI355X", section "FP8 Error in
Full-Model Inference" and footnote 2: Q, K and V are quantized to e4m3 before
attention, Q in a pass of its own (with the rotation fused in) and K, V as they
are written to the KV cache; an optional Hadamard rotation of Q and K over the
head dimension leaves Q K^T unchanged and spreads outlier channels.

The pages do not give the scale granularity or formula. The readings used here:

* one float32 scale per (batch, head, block of ``block`` consecutive tokens),
  shared by all head-dim channels; the last block may be shorter;
* amax = max |x| over the block; s = the smallest power of two with
  amax / s <= 448 (at least 2^-126, a normal float32), or s = 1 when amax == 0 (absmax scaling with the zero guard
  of the FP8 GEMM on CDNA4 blog, section 2.2, with the scale restricted to a
  power of two, the E8M0 form that the ZYFA page's scaled FP8 matrix
  instruction applies exactly: section "Per-Block Scaling and Normalization by
  the Rounded Row Sum");
* code = e4m3(x / s): the quotient is exact (s is a power of two), then
  round-to-nearest-even to e4m3 with saturation (blog section 2.3).

The e4m3 grid is the same in every binade, so a power-of-two scale gives the
same relative precision to all normal values as amax / 448 would; the largest
element lands in (224, 448]. The dequantized value of an element is
decode(code) * s, exact in float64.
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
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float64)  # exact: a max of float32 magnitudes
        s = np.ones(amax.shape)
        nz = amax > 0
        k = np.ceil(np.log2(amax[nz] / E4M3_MAX))
        # make k exactly the least integer with amax <= 448 * 2^k (guards log2 rounding)
        k = np.where(amax[nz] > E4M3_MAX * np.exp2(k), k + 1, k)
        k = np.where(amax[nz] <= E4M3_MAX * np.exp2(k - 1), k - 1, k)
        s[nz] = np.exp2(np.maximum(k, -126))  # keep the scale a normal float32
        s = s.astype(np.float32)
        y = blk.astype(np.float64) / s[:, :, None, None]  # exact: division by a power of two
        codes[:, :, j * block:(j + 1) * block, :] = e4m3_encode(y)
        scales[:, :, j] = s
    return codes, scales


def dequantize_blocks(codes, scales, block):
    """Float64 values decode(code) * scale for codes [B, H, S, D] and scales [B, H, nb]."""
    codes = np.asarray(codes)
    S = codes.shape[2]
    per_token = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :S]
    return e4m3_decode(codes) * per_token[..., None]


def paley_hadamard_12():
    """Hadamard matrix of order 12 from Paley's first construction over GF(11) (11 = 3 mod 4):
    chi is the quadratic character of GF(11) (chi(0) = 0, +1 on the nonzero squares, -1
    elsewhere), Q[i][j] = chi(j - i) its Jacobsthal matrix, S the 12 x 12 matrix with a zero
    corner, ones along the rest of the first row, minus ones down the rest of the first
    column and Q below and to the right; H = I + S. Entries +-1, H H^T = 12 I."""
    q = 11
    squares = {(x * x) % q for x in range(1, q)}

    def chi(x):
        x %= q
        return 0 if x == 0 else (1 if x in squares else -1)

    s = np.zeros((12, 12))
    s[0, 1:] = 1.0
    s[1:, 0] = -1.0
    s[1:, 1:] = [[chi(j - i) for j in range(q)] for i in range(q)]
    return np.eye(12) + s


def hadamard_matrix(n):
    """Hadamard matrix of order n, entries +-1, unnormalized.

    n a power of two: Sylvester's H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]].
    n = 12 * 2^k (192 for the MLA head dimension): the Kronecker product of the order-12
    Paley matrix and the Sylvester matrix of order 2^k, element (m 2^k + b, m' 2^k + b') =
    P12[m, m'] * H[b, b'], itself a Hadamard matrix of order n."""
    if n >= 1 and not n & (n - 1):
        h = np.ones((1, 1))
        while h.shape[0] < n:
            h = np.block([[h, h], [h, -h]])
        return h
    if n % 12 == 0 and n >= 12 and not (n // 12) & (n // 12 - 1):
        return np.kron(paley_hadamard_12(), hadamard_matrix(n // 12))
    raise ValueError("order must be a power of two or 12 times one")


def hadamard_rotate(x):
    """Rotate the last axis of ``x`` by the orthonormal Hadamard matrix H_n / sqrt(n),
    in float64: y = x @ (H_n / sqrt(n)), a row vector times the matrix (for powers of two
    H_n is symmetric; the order-192 matrix is not). Rotating both Q and K leaves Q K^T
    unchanged (H H^T = n I)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    return x @ (hadamard_matrix(n) / np.sqrt(n))
