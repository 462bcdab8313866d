"""Pins for the oracle's block quantizer and Hadamard rotation.

Pinned by: the absmax definition (the largest element lands on the top code),
the zero guard, the e4m3 error bound, torch's float8_e4m3fn cast of the same
float32 quotients (a library routine), SciPy's Hadamard matrix (a library
routine) and the orthogonality that makes Q K^T invariant.
"""

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import (quantize_blocks, dequantize_blocks, hadamard_matrix, hadamard_rotate, e4m3_decode,
                    paley_hadamard_12)


def _x(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("S", [128, 200, 64, 1])
def test_scale_is_least_power_of_two_over_absmax(block, S):
    x = _x((2, 3, S, 128)) * np.float32(3.7)
    codes, scales = quantize_blocks(x, block)
    nb = (S + block - 1) // block
    assert scales.shape == (2, 3, nb) and scales.dtype == np.float32
    m, e = np.frexp(scales.astype(np.float64))
    assert np.all(m == 0.5)  # powers of two
    for j in range(nb):
        amax = np.abs(x[:, :, j * block:(j + 1) * block]).max(axis=(2, 3)).astype(np.float64)
        s = scales[:, :, j].astype(np.float64)
        assert np.all(amax / s <= 448.0) and np.all(amax / s > 224.0)  # the least such power of two
        # the largest-magnitude element of each block is coded with the exact quotient's rounding
        blk = x[:, :, j * block:(j + 1) * block]
        for b in range(2):
            for h in range(3):
                i = np.unravel_index(np.argmax(np.abs(blk[b, h])), blk[b, h].shape)
                c = codes[b, h, j * block + i[0], i[1]]
                assert abs(e4m3_decode(c)) >= 224.0


def test_tiny_and_huge_blocks():
    x = np.zeros((1, 1, 192, 128), np.float32)
    x[0, 0, :64, 0] = 1e-42           # denormal float32: the scale stays at 2^-126
    x[0, 0, 64:128, 3] = 3.0e38
    x[0, 0, 128:, 5] = 448.0           # exactly 448 * 2^0
    codes, scales = quantize_blocks(x, 64)
    assert scales[0, 0, 0] == np.float32(2.0 ** -126)
    assert scales[0, 0, 1] == np.float32(2.0 ** 120) and 3.0e38 / 2.0 ** 120 <= 448
    assert scales[0, 0, 2] == 1.0 and codes[0, 0, 128, 5] == 0x7E


def test_zero_block_guard():
    x = _x((1, 1, 128, 128))
    x[:, :, :64] = 0.0
    codes, scales = quantize_blocks(x, 64)
    assert scales[0, 0, 0] == 1.0
    assert np.all(codes[0, 0, :64] == 0)
    assert scales[0, 0, 1] != 1.0


def test_dequantization_error_bound():
    x = _x((1, 2, 256, 128), seed=1)
    codes, scales = quantize_blocks(x, 128)
    xd = dequantize_blocks(codes, scales, 128)
    s = np.repeat(scales.astype(np.float64), 128, axis=2)[..., None]
    y = np.abs(x / s)
    err = np.abs(xd - x) / s
    normal = y >= 2.0 ** -6
    # 3 mantissa bits: relative error at most 2^-4 (half an ulp) plus the float32 quotient's rounding
    assert np.all(err[normal] <= y[normal] * (2.0 ** -4) * (1 + 1e-5))
    # subnormal range: absolute error at most half the subnormal spacing 2^-9
    assert np.all(err[~normal] <= 2.0 ** -10 * (1 + 1e-5))


def test_codes_match_torch_cast_of_quotients():
    x = _x((1, 4, 192, 128), seed=2) * np.float32(3.0)
    codes, scales = quantize_blocks(x, 64)
    s = np.repeat(scales, 64, axis=2)[:, :, :192, None]
    q = (torch.from_numpy(x) / torch.from_numpy(s)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, q)


def test_hadamard_matches_scipy_and_is_orthogonal():
    for n in [1, 2, 4, 8, 64, 128]:
        h = hadamard_matrix(n)
        assert np.array_equal(h, scipy.linalg.hadamard(n))
        assert np.array_equal(h @ h.T, n * np.eye(n))
    for n in (6, 20, 100, 200):
        with pytest.raises(ValueError):
            hadamard_matrix(n)


@pytest.mark.parametrize("n", [12, 24, 192])
def test_order_12_times_power_of_two_is_hadamard(n):
    # the defining properties: entries +-1 and mutually orthogonal rows (H H^T = n I), so
    # H / sqrt(n) is orthonormal; a Paley matrix of order 12 has a first row of ones
    h = hadamard_matrix(n)
    assert set(np.unique(h)) == {-1.0, 1.0}
    assert np.array_equal(h @ h.T, n * np.eye(n))
    assert np.array_equal(h.T @ h, n * np.eye(n))
    p12 = paley_hadamard_12()
    assert np.array_equal(p12[0], np.ones(12)) and np.array_equal(p12 @ p12.T, 12 * np.eye(12))
    # not a Sylvester matrix in disguise: no power-of-two Hadamard matrix has order 12
    assert not np.array_equal(p12, p12.T)


def test_order_192_rotation_preserves_scores_and_spreads_outliers():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((40, 192))
    k = rng.standard_normal((40, 192))
    q[:, 150] *= 15
    k[:, 150] *= 15
    qr, kr = hadamard_rotate(q), hadamard_rotate(k)
    assert np.allclose(qr @ kr.T, q @ k.T, rtol=0, atol=1e-10)
    assert np.allclose(np.linalg.norm(qr, axis=1), np.linalg.norm(q, axis=1), rtol=1e-12)
    for j in (0, 17, 150, 191):
        e = np.zeros(192)
        e[j] = 1.0
        assert np.allclose(np.abs(hadamard_rotate(e)), 1 / np.sqrt(192))
    assert np.abs(kr).max() < np.abs(k).max() / 3


def test_hadamard_rotation_preserves_scores_and_spreads_outliers():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((64, 128))
    k = rng.standard_normal((64, 128))
    q[:, 7] *= 15
    k[:, 7] *= 15
    qr, kr = hadamard_rotate(q), hadamard_rotate(k)
    assert np.allclose(qr @ kr.T, q @ k.T, rtol=0, atol=1e-10)
    # a single outlier channel is spread evenly over all 128 channels
    e = np.zeros(128)
    e[7] = 1.0
    assert np.allclose(np.abs(hadamard_rotate(e)), 1 / np.sqrt(128))
    assert np.abs(kr).max() < np.abs(k).max() / 3


def _torch_decode(codes):
    """e4m3 values of codes through torch's float8_e4m3fn (a library routine), float64."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _varying_scales(B, H, nb, seed):
    """Scales that differ from block to block: 2^(j mod 5) times a seeded factor in [1, 2)
    (not only powers of two: the attention entry points accept any positive scale)."""
    rng = np.random.default_rng(seed)
    j = np.arange(nb)[None, None, :]
    return (np.exp2(j % 5) * rng.uniform(1.0, 2.0, (B, H, nb))).astype(np.float32)


def _dequantize_rolled(codes, scales, block):
    """A planted mistake: block j takes block j-1's scale."""
    return dequantize_blocks(codes, np.roll(scales, 1, axis=2), block)


@pytest.mark.parametrize("block,S", [(64, 200), (128, 300), (64, 64), (128, 129)])
def test_dequantize_applies_each_blocks_own_scale(block, S):
    # "Error of a Single Attention Call" (ZYFA): the reference attends over the dequantized
    # inputs the kernel read, element = decode(code) * scale of the element's token block.
    # Checked element by element against torch's decode of every code, the block found by
    # explicit division of the token index, the last block ragged (S not a multiple of it).
    rng = np.random.default_rng(block + S)
    codes = rng.integers(0, 256, (2, 3, S, 16)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    nb = (S + block - 1) // block
    scales = _varying_scales(2, 3, nb, seed=S)
    got = dequantize_blocks(codes, scales, block)
    vals = _torch_decode(codes)
    want = np.empty_like(vals)
    for t in range(S):
        want[:, :, t, :] = vals[:, :, t, :] * scales[:, :, t // block, None].astype(np.float64)
    assert got.dtype == np.float64 and got.shape == codes.shape
    assert np.array_equal(got, want)
    # the same comparison catches a scale taken from the neighbouring block
    if nb > 1:
        assert not np.array_equal(_dequantize_rolled(codes, scales, block), want)


@pytest.mark.parametrize("block", [64, 128])
def test_quantize_round_trip_with_block_varying_magnitudes(block):
    # token block j is scaled by 2^(3 (j mod 5)): each block's scale tracks its own absmax,
    # and every dequantized element is within e4m3's bound of its own block's scale
    S = 5 * block + 37
    x = _x((1, 2, S, 128), seed=block)
    mag = np.exp2(3.0 * ((np.arange(S) // block) % 5)).astype(np.float32)
    x = x * mag[None, None, :, None]
    codes, scales = quantize_blocks(x, block)
    for j in range(scales.shape[2]):
        amax = np.abs(x[:, :, j * block:(j + 1) * block]).max(axis=(2, 3)).astype(np.float64)
        assert np.all(amax / scales[:, :, j] <= 448.0) and np.all(amax / scales[:, :, j] > 224.0)
    xd = dequantize_blocks(codes, scales, block)
    s = np.repeat(scales.astype(np.float64), block, axis=2)[:, :, :S, None]
    assert np.all(np.abs(xd - x) <= np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-5))
    # a rolled scale puts whole blocks off by a factor of 8 or more
    xr = _dequantize_rolled(codes, scales, block)
    assert np.max(np.abs(xr - x) / (np.abs(x) + s)) > 1.0
