"""Pins for the oracle's e4m3 codec and bf16 helpers (CPU only).

The codec is checked against the OCP e4m3fn format's fixed points, against
torch's CPU float8_e4m3fn cast (an independent library routine) on every
midpoint and random values, and for round-trip and monotonicity.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3


# Fixed points of OCP e4m3fn: (code, value).
FIXED = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x77, 240.0),
    (0x7E, 448.0), (0x81, -(2.0 ** -9)), (0xB8, -1.0), (0xFE, -448.0),
]


@pytest.mark.parametrize("code,value", FIXED)
def test_decode_fixed_points(code, value):
    assert e4m3.decode_one(code) == value


def test_decode_nan_and_negative_zero():
    assert math.isnan(e4m3.decode_one(0x7F)) and math.isnan(e4m3.decode_one(0xFF))
    assert e4m3.decode_one(0x80) == 0.0 and math.copysign(1.0, e4m3.decode_one(0x80)) == -1.0


def test_decode_matches_torch_table():
    ours = e4m3.decode_table()
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(theirs)
    assert np.array_equal(ours[~both_nan], theirs[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))


def test_roundtrip_and_monotone():
    codes = np.array([c for c in range(256) if c not in e4m3.NAN_CODES], dtype=np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode_rne(vals), codes)
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def _torch_encode(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_midpoints():
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact in fp32
    probes = [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)), pos.astype(np.float32)]
    v = np.concatenate(probes)
    v = np.concatenate([v, -v])
    assert np.array_equal(e4m3.encode_rne(v), _torch_encode(v))


def test_encode_matches_torch_random():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.uniform(-460, 460, 200_000),
        rng.standard_normal(200_000) * 3,
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 100_000),
        rng.uniform(-2.0 ** -10, 2.0 ** -10, 50_000),
    ]).astype(np.float32)
    assert np.array_equal(e4m3.encode_rne(v), _torch_encode(v))


def test_ties_to_even_examples():
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): even code wins.
    assert e4m3.encode_rne([1.0625])[0] == 0x38
    assert e4m3.encode_rne([1.1875])[0] == 0x3A  # between 1.125 and 1.25
    assert e4m3.encode_rne([17.0])[0] == e4m3.encode_rne([16.0])[0]
    assert e4m3.encode_rne([19.0])[0] == e4m3.encode_rne([20.0])[0]
    # smallest subnormal halfway: 2^-10 ties to 0
    assert e4m3.encode_rne([2.0 ** -10])[0] == 0x00
    assert e4m3.encode_rne([3 * 2.0 ** -10])[0] == 0x02


def test_sign_and_saturation_reading():
    assert e4m3.encode_rne([-0.0])[0] == 0x80
    assert e4m3.encode_rne([-1e-30])[0] == 0x80  # rounds to zero, keeps the sign
    assert e4m3.encode_rne([450.0])[0] == 0x7E
    assert e4m3.encode_rne([1e6])[0] == 0x7E  # satfinite reading
    assert e4m3.encode_rne([-1e6])[0] == 0xFE
    with pytest.raises(ValueError):
        e4m3.encode_rne([np.nan])


def test_bf16_widen_and_round():
    x = torch.randn(10000, dtype=torch.float32)
    b = x.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.to_f32(bits), b.to(torch.float32).numpy())
    # On fp32-representable values torch's cast rounds once, so it must agree.
    rng = np.random.default_rng(3)
    d = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        (1 + (2 * np.arange(0, 64) + 1) * 2.0 ** -8)])  # exact bf16 ties
    d = d.astype(np.float32).astype(np.float64)
    ours = bf16.bits_from_f64(d)
    theirs = torch.from_numpy(d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def _nearest_bf16_exact(v):
    """Nearest bf16 to fp64 v by exact rational comparison of the two neighbours."""
    f = np.float32(v)  # a neighbour candidate region; search bf16 patterns around it
    base = int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)
    cands = [(base + d) & 0xFFFF for d in (-1, 0, 1, 2)]
    vals = [Fraction(float(bf16.to_f32(np.array([c], dtype=np.uint16))[0])) for c in cands]
    fv = Fraction(v)
    best = min(range(4), key=lambda i: (abs(vals[i] - fv), cands[i] & 1))
    return cands[best]


def test_bf16_round_f64_single_rounding():
    # General fp64 values: compare with exact rational nearest-even.  torch's
    # fp64 -> bf16 cast goes through fp32 and double-rounds, so it is not used.
    rng = np.random.default_rng(5)
    d = rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000)
    ours = bf16.bits_from_f64(d)
    for v, o in zip(d, ours):
        assert o == _nearest_bf16_exact(float(v)), v
    # The double-rounding case found by comparing with torch: -6.752998179955093e-11
    # lies just past the midpoint of its two bf16 neighbours.
    assert bf16.bits_from_f64([-6.752998179955093e-11])[0] == 0xAE95


def test_bf16_round_exact_ties():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert bf16.round_f64([1 + 2.0 ** -8])[0] == 1.0
    assert bf16.round_f64([1 + 3 * 2.0 ** -8])[0] == 1 + 2 * 2.0 ** -7
    # exactness check against a Fraction computation
    v = 1.2345678
    r = bf16.round_f64([v])[0]
    assert abs(Fraction(r) - Fraction(v)) <= Fraction(1, 2 ** 8)
