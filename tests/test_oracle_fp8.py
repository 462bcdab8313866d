"""Pins for the oracle's e4m3 and bfloat16 codecs.

Pinned by: the code points and thresholds the pages print (tests/golden/
e4m3_printed.json), the exhaustive decode of all 256 codes against torch's
float8_e4m3fn casts, round-to-nearest-even tie cases, saturation, and torch's
bfloat16 cast (a library routine).
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode, bf16_round, f32_to_bf16_bits, E4M3_MAX

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_printed.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_printed_code_points(golden):
    for value, code in golden["codes"]["value_to_code"]:
        assert int(e4m3_encode(np.float32(value))) == code
        assert e4m3_decode(code) == value
    for code, value in golden["codes"]["code_to_value"]:
        assert e4m3_decode(code) == value
    # the code grows by 8 per doubling across every normal binade
    step = golden["codes"]["code_step_per_doubling"]
    for e in range(-6, 8):
        assert int(e4m3_encode(2.0 ** (e + 1))) - int(e4m3_encode(2.0 ** e)) == step


def test_printed_thresholds(golden):
    t = golden["thresholds"]
    smallest_normal = t["smallest_normal"]
    # smallest normal is exactly representable with full mantissa: the next value up is 1/8 ulp higher
    c = int(e4m3_encode(smallest_normal))
    assert e4m3_decode(c) == smallest_normal
    assert e4m3_decode(c + 1) == smallest_normal * (1 + 2.0 ** -t["mantissa_bits"])
    # below the smallest normal, spacing stays 2^-9 (subnormals): fewer significant bits
    assert e4m3_decode(c - 1) == smallest_normal - 2.0 ** -9
    # values below 2^-10 round to zero; just above it they round to the smallest subnormal 2^-9
    u = t["underflow_below"]
    assert int(e4m3_encode(u * 0.999)) == 0
    assert int(e4m3_encode(u * 1.001)) == 1
    assert int(e4m3_encode(u)) == 0  # exact tie between 0 and 2^-9: even code 0
    r = golden["range"]
    assert e4m3_decode(0x7E) == r["e4m3_max"] == E4M3_MAX
    assert r["e4m3_min_normal"] == smallest_normal


def test_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], theirs[~nan])


def test_encode_against_torch_in_range():
    rng = np.random.default_rng(7)
    vals = e4m3_decode(np.arange(127))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([
        vals, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.6, 20000),
    ]).astype(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448.0]  # torch does not saturate; compare inside the finite range
    ours = e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_round_half_to_even():
    # 1.0 (code 56) and 1.125 (code 57): the midpoint goes to the even code 56;
    # 1.125 and 1.25 (58): the midpoint goes to 58
    assert int(e4m3_encode(1.0625)) == 56
    assert int(e4m3_encode(1.1875)) == 58
    assert int(e4m3_encode(np.nextafter(np.float32(1.0625), np.float32(2)))) == 57


def test_saturation_and_signs():
    assert int(e4m3_encode(1e6)) == 0x7E
    assert int(e4m3_encode(-1e6)) == 0xFE
    assert int(e4m3_encode(np.inf)) == 0x7E
    assert int(e4m3_encode(460.0)) == 0x7E
    assert int(e4m3_encode(-0.0)) == 0x80
    assert int(e4m3_encode(-1e-6)) == 0x80
    assert int(e4m3_encode(np.nan)) == 0x7F


def test_bf16_round_against_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000)).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, bits[np.isfinite(bits)], np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875])])
    ours = f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(ours, theirs)
    assert np.array_equal(bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())
