"""Test plumbing shared by the GPU tests: run the HIP path through the binding and the
oracle on the same seeded inputs, and compare.

The two sides share nothing but the input arrays: the GPU side uploads the float32
inputs and runs the library's quantizer and attention kernels; the oracle side runs
oracle.quantize_blocks / hadamard_rotate / causal_attention on the host."""

import math

import numpy as np
import torch

import fp8_causal_prefill_amd as zy
from oracle import (causal_attention, dequantize_blocks, hadamard_rotate, quantize_blocks, bf16_bits_to_f64,
                    f32_to_bf16_bits)

DEV = "cuda"


def rel_l2(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def bf16_from_f64(t: torch.Tensor):
    return t.float().cpu().numpy().astype(np.float64)


# ---------------- GPU side ----------------

# float32 error of the kernels' rotation, as a multiple of 2^-24 * sum |x| / sqrt(D) over the
# row: the order-128 transform is 7 butterfly stages and the scaling (at most 9 roundings
# along any path, each bounded by the sum of the magnitudes it adds); the order-192 product
# is 4 stages of H_16 and the order-12 sums (at most 8 roundings deep, over terms bounded by
# three times the row's magnitude sum), about 30. One bound serves both.
ROTATION_NOISE_ULPS = 32


def rotation_noise(x, scales, block):
    """Per-element bound on |t32 - t| for codes of a rotated x [B, H, S, D] with block scales
    [B, H, nb]: t is the exact rotated value over its scale, t32 the kernel's float32 one."""
    S, D = x.shape[2], x.shape[3]
    row = np.abs(x.astype(np.float64)).sum(axis=-1, keepdims=True)
    s = np.repeat(scales.astype(np.float64), block, axis=2)[:, :, :S, None]
    return ROTATION_NOISE_ULPS * 2.0 ** -24 * row / math.sqrt(D) / s


def gpu_quantize(x, block, hadamard=False):
    codes, scales = zy.quantize_fp8(to_dev(x), block, hadamard)
    return codes, scales


def gpu_fp8(q, k, v, block, hadamard=False, scale=None, return_lse=True, lean=False):
    """fp32 numpy inputs -> GPU quantizer -> GPU FP8 attention (exact or lean
    probabilities). Returns numpy (o float64, lse float64, (qc, qs, kc, ks, vc, vs) numpy)."""
    qc, qs = gpu_quantize(q, block, hadamard)
    kc, ks = gpu_quantize(k, block, hadamard)
    vc, vs = gpu_quantize(v, block, False)
    o, lse = zy.attn_fwd_fp8(qc, kc, vc, qs, ks, vs, block, scale, return_lse=return_lse, lean=lean)
    torch.cuda.synchronize()
    parts = tuple(t.cpu().numpy() for t in (qc, qs, kc, ks, vc, vs))
    return bf16_from_f64(o), (lse.cpu().numpy().astype(np.float64) if lse is not None else None), parts


def gpu_bf16(q, k, v, scale=None, return_lse=True):
    """fp32 numpy inputs -> torch's bfloat16 cast (host) -> GPU BF16 attention."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(DEV)
    o, lse = zy.attn_fwd_bf16(t(q), t(k), t(v), scale, return_lse=return_lse)
    torch.cuda.synchronize()
    return bf16_from_f64(o), (lse.cpu().numpy().astype(np.float64) if lse is not None else None)


# ---------------- oracle side ----------------

def oracle_inputs_fp8(q, k, v, block, hadamard=False):
    if hadamard:
        q = hadamard_rotate(q).astype(np.float32)
        k = hadamard_rotate(k).astype(np.float32)
    qc, qs = quantize_blocks(q, block)
    kc, ks = quantize_blocks(k, block)
    vc, vs = quantize_blocks(v, block)
    return (qc, qs, kc, ks, vc, vs)


def oracle_attention_from_codes(parts, block, scale, rows=None):
    qc, qs, kc, ks, vc, vs = parts
    return causal_attention(dequantize_blocks(qc, qs, block), dequantize_blocks(kc, ks, block),
                            dequantize_blocks(vc, vs, block), scale, rows=rows)


def oracle_bf16(q, k, v, scale, rows=None):
    qb, kb, vb = (f32_to_bf16_bits(x) for x in (q, k, v))
    o, lse = causal_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), scale, rows=rows)
    return o, lse, (qb, kb, vb)


def default_scale(d):
    return 1.0 / math.sqrt(d)
