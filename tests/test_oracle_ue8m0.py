"""Pins for the oracle's power-of-two (UE8M0) quantisers (CPU only).

Checked against things other than the quantiser itself: the exponent against
the defining inequalities 2^(E-128) < amax/448 <= 2^(E-127) evaluated in
exact rational arithmetic and against math.frexp on the fp64 quotient; the
codes against torch's CPU float8_e4m3fn cast of the exactly scaled values;
the case where amax/448 is itself a power of two against the fp32-scale
quantiser (the two definitions coincide there); zero tiles; the e4m3 range
of every scaled value; and the layouts.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, quant, ue8m0
from synth import bf16_normal


def _bf16_bits(values):
    t = torch.tensor(values, dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("amax", [448.0, 447.0, 449.0, 1.0, 0.5, 3.0, 7.0 * 2 ** -10, 2.0 ** -100, 3.0e38, 1e-30])
def test_exponent_is_the_smallest_power_of_two(amax):
    a = float(bf16.to_f32(_bf16_bits([amax]))[0])
    e = ue8m0.exponent(a)
    r = Fraction(a) / 448
    assert 0 <= e <= 254
    if 0 < e:
        assert Fraction(2) ** (e - 127) >= r
        assert Fraction(2) ** (e - 128) < r
    # frexp route on the fp64 quotient (exact enough: no bf16 amax puts
    # amax/448 within 2^-53 of a power of two unless it is one)
    m, x = math.frexp(a / 448.0)
    assert e == min(254, max(0, (x - 1 if m == 0.5 else x) + 127))


def test_exponent_zero_and_clamp():
    assert ue8m0.exponent(0.0) == 0
    tiny = float(bf16.to_f32(np.array([1], dtype=np.uint16))[0])  # smallest bf16 subnormal
    assert ue8m0.exponent(tiny) == 0                               # 2^-133/448 is below 2^-127
    big = float(bf16.to_f32(np.array([0x7F7F], dtype=np.uint16))[0])
    assert ue8m0.exponent(big) == 127 + math.ceil(math.log2(big / 448))


@pytest.mark.parametrize("rows,cols", [(1, 128), (7, 256), (33, 384)])
def test_1x128_codes_match_torch_cast_of_scaled_values(rows, cols):
    x = bf16_normal((rows, cols), seed=71 + rows, scale=3.0)
    q, sf = ue8m0.quant_1x128_ue8m0(x)
    ld = (rows + 3) // 4 * 4
    assert sf.shape == (cols // 128, ld) and sf.dtype == np.uint8 and np.all(sf[:, rows:] == 0)
    xf = bf16.to_f32(x).astype(np.float64)
    for j in range(cols // 128):
        e = sf[j, :rows].astype(np.int64)
        scaled = xf[:, j * 128:(j + 1) * 128] * np.ldexp(1.0, 127 - e)[:, None]
        assert np.all(np.abs(scaled) <= 448.0)
        ref = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q[:, j * 128:(j + 1) * 128], ref)
        amax = np.abs(xf[:, j * 128:(j + 1) * 128]).max(axis=1)
        assert all(e[r] == ue8m0.exponent(amax[r]) for r in range(rows))


def test_power_of_two_ratio_coincides_with_fp32_scales():
    # amax = 448 * 2^j exactly: the fp32 rule gives s = 2^j too, so codes and
    # scales must agree with the fp32-scale quantiser element for element.
    rng = np.random.default_rng(5)
    rows = 6
    x = rng.standard_normal((rows, 256)).astype(np.float32)
    x = np.clip(x, -3, 3)
    for r in range(rows):
        j = [-6, -2, 0, 1, 3, 7][r]
        x[r] *= (448.0 * 2.0 ** j) / 3.0 * 0.5
        x[r, 0] = 448.0 * 2.0 ** j
        x[r, 128] = -448.0 * 2.0 ** j
    bits = _bf16_bits(x)
    q8, e = ue8m0.quant_1x128_ue8m0(bits)
    q32, s32 = quant.quant_1x128(bits)
    assert np.array_equal(q8, q32)
    assert np.array_equal(ue8m0.scale_of(e[:, :rows]).astype(np.float32), s32[:, :rows])


def test_zero_tile_keeps_signed_zeros():
    bits = np.zeros((2, 128), dtype=np.uint16)
    bits[1, ::2] = 0x8000
    q, sf = ue8m0.quant_1x128_ue8m0(bits)
    assert np.all(sf[0, :2] == 0)
    assert np.all(q[0] == 0) and np.all(q[1, ::2] == 0x80) and np.all(q[1, 1::2] == 0)


def test_128x128_layout_partial_block_and_codes():
    n, k = 200, 384
    w = bf16_normal((n, k), seed=91, scale=0.01)
    q, sf = ue8m0.quant_128x128_ue8m0(w)
    nb = 2
    assert sf.shape == (k // 128, 4) and np.all(sf[:, nb:] == 0)
    wf = bf16.to_f32(w).astype(np.float64)
    for i in range(nb):
        r0, r1 = i * 128, min(n, (i + 1) * 128)
        for j in range(k // 128):
            blk = wf[r0:r1, j * 128:(j + 1) * 128]
            e = int(sf[j, i])
            assert e == ue8m0.exponent(float(np.abs(blk).max()))
            scaled = (blk * 2.0 ** (127 - e)).astype(np.float32)
            ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[r0:r1, j * 128:(j + 1) * 128], ref)
    s = ue8m0.sfb_as_fp32(sf, n)
    assert s.shape == (nb, k // 128)
    assert np.array_equal(s, np.ldexp(1.0, sf[:, :nb].T.astype(np.int64) - 127).astype(np.float32))
