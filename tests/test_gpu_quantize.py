"""GPU quantizer (zyfa_quantize_fp8) against the oracle's block quantizer.

Without rotation the codes and scales are an integer / exactly-rounded result and
must match bit for bit. With the Hadamard rotation the GPU rotates in float32 by a
fast Walsh-Hadamard transform while the oracle rotates in float64, so a code may
differ where the rotated value sits on a rounding boundary, and a power-of-two
scale where the block absmax sits on a binade boundary: every GPU code must still
be a correct rounding of the oracle's exactly rotated value (over the GPU's scale)
up to float32 noise."""

import numpy as np
import pytest
import torch

import fp8_causal_prefill_amd as zy
from oracle import quantize_blocks, hadamard_rotate, e4m3_decode
from workloads import custom, generate
from tests.paths import gpu_quantize, rotation_noise, to_dev

pytestmark = pytest.mark.gpu


def _print_case(**kw):
    print("case:", ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


@pytest.mark.parametrize("S", [128, 1, 63, 64, 65, 300, 1000])
@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("D", [128, 192])
def test_quantize_bit_exact_fp32(S, block, D):
    _print_case(S=S, block=block, D=D)
    x, _, _ = generate(custom(2, 3, 3, S, D, D, wid=200 + S), seed=1)
    x = x * np.float32(2.5)
    codes, scales = gpu_quantize(x, block)
    rc, rs = quantize_blocks(x, block)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_bit_exact_bf16_input():
    x, _, _ = generate(custom(1, 4, 4, 257, 128, 128, wid=301), seed=2)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    codes, scales = __import__("fp8_causal_prefill_amd").quantize_fp8(xb.to("cuda"), 128)
    rc, rs = quantize_blocks(xb.float().numpy(), 128)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_zero_block_and_extremes():
    x = np.zeros((1, 1, 256, 128), np.float32)
    x[0, 0, 128:] = np.random.default_rng(3).standard_normal((128, 128)).astype(np.float32) * 1e-30
    x[0, 0, 200, 5] = 3e38
    codes, scales = gpu_quantize(x, 64)
    rc, rs = quantize_blocks(x, 64)
    assert scales[0, 0, 0].item() == 1.0
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("S,block,D", [(128, 64, 128), (333, 128, 128), (128, 64, 192), (333, 128, 192),
                                       (64, 128, 192)])
def test_quantize_hadamard(S, block, D):
    _print_case(S=S, block=block, D=D)
    w = custom(1, 2, 2, S, D, 128, dist="activation", wid=400 + S)
    x, _, _ = generate(w, seed=4)
    codes, scales = gpu_quantize(x, block, hadamard=True)
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    y = hadamard_rotate(x)  # exact rotation (float64)
    rc, rs = quantize_blocks(y.astype(np.float32), block)
    # scales: powers of two from the block absmax of a float32-computed rotation; they can
    # differ from the exact rotation's only where that absmax sits on a binade boundary
    ratio = scales.astype(np.float64) / rs
    assert np.all((ratio == 1.0) | (ratio == 2.0) | (ratio == 0.5))
    assert np.mean(ratio != 1.0) < 0.05
    # every GPU code decodes to a nearest e4m3 value of y / s up to float32 noise in y
    s = np.repeat(scales.astype(np.float64), block, axis=2)[:, :, :S, None]
    t = y / s
    noise = rotation_noise(x, scales, block)  # the kernel's float32 rotation error, in code units
    dec = e4m3_decode(codes)
    err = np.abs(dec - t)
    half_ulp = np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10)
    # (half a step of the kernel's float32 value t32 is at most half a step of t plus 2^-4 of
    # |t32 - t|; 2^-20 |t| covers the roundings of the scale product)
    assert np.all(err <= half_ulp + noise * (1 + 2.0 ** -4) + np.abs(t) * 2.0 ** -20)
    mismatch = np.mean(codes != rc)
    assert mismatch < 1e-3, mismatch


@pytest.mark.parametrize("D,block,S", [(128, 64, 200), (192, 64, 200), (128, 128, 333), (192, 128, 333),
                                       (192, 128, 17)])
def test_quantize_hadamard_bf16_input(D, block, S):
    # the bfloat16-input rotation paths (D = 128: the fast Walsh-Hadamard transform; D = 192:
    # the Paley-Sylvester product, whose bfloat16 rows come in through LDS): every code a
    # nearest e4m3 value of the exact rotation of the bfloat16 values the kernel read, divided
    # by the block's power-of-two scale; ragged last blocks (8, 77 and 17 rows of a block)
    _print_case(D=D, block=block, S=S, bf16=True)
    w = custom(1, 3, 3, S, D, 128, dist="activation", wid=470 + D + S)
    x, _, _ = generate(w, seed=5)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    codes, scales = zy.quantize_fp8(xb.to("cuda"), block, True)
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    y = hadamard_rotate(xb.float().numpy())  # the bf16 values the kernel read, rotated exactly
    m, _ = np.frexp(scales.astype(np.float64))
    assert np.all(m == 0.5)
    s = np.repeat(scales.astype(np.float64), block, axis=2)[:, :, :S, None]
    t = y / s
    noise = rotation_noise(xb.float().numpy(), scales, block)  # float32 rotation error, in code units
    err = np.abs(e4m3_decode(codes) - t)
    half_ulp = np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10)
    # (half a step of the kernel's float32 value t32 is at most half a step of t plus 2^-4 of
    # |t32 - t|; 2^-20 |t| covers the roundings of the scale product)
    assert np.all(err <= half_ulp + noise * (1 + 2.0 ** -4) + np.abs(t) * 2.0 ** -20)
    # the scale is the least power of two that holds the block's rotated absmax (up to the
    # float32 rotation's noise at a binade boundary)
    for j in range(scales.shape[2]):
        r = np.abs(y[:, :, block * j:block * (j + 1)]).max(axis=(2, 3)) / scales[:, :, j]
        assert np.all(r <= 448 * (1 + 1e-6)) and np.all(r > 224 * (1 - 1e-6))
