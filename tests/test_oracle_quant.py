"""Pins for the oracle's 1x128 and 128x128 quantisers (CPU only).

Checked against things other than the quantiser itself: the e4m3 step
against torch's CPU float8_e4m3fn cast, the fp32 scale and quotient against
correctly rounded fp64 arithmetic (dividing in fp64 and rounding to fp32 is
innocuous for division), and invariants that any correct amax/448 quantiser
satisfies (a +-448 code at the amax element, the dequantisation error bound,
power-of-two invariance, zero tiles, layout of the scale matrices).
"""

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, quant
from synth import bf16_normal


def _f32(bits):
    return bf16.to_f32(bits)


def _scale_fp64_route(amax):
    return np.float32(float(amax) / 448.0)


@pytest.mark.parametrize("rows,cols", [(1, 128), (5, 256), (33, 384), (64, 7168)])
def test_1x128_layout_and_scales(rows, cols):
    x = bf16_normal((rows, cols), seed=11 + rows)
    q, sf = quant.quant_1x128(x)
    ld = (rows + 3) // 4 * 4
    assert q.shape == (rows, cols) and q.dtype == np.uint8
    assert sf.shape == (cols // 128, ld) and sf.dtype == np.float32
    assert np.all(sf[:, rows:] == 0)
    xf = _f32(x).reshape(rows, cols // 128, 128)
    amax = np.abs(xf).max(axis=2)
    for r in range(rows):
        for j in range(cols // 128):
            assert sf[j, r] == _scale_fp64_route(amax[r, j])


def test_1x128_codes_match_torch_cast_of_quotient():
    x = bf16_normal((48, 1024), seed=21)
    q, sf = quant.quant_1x128(x)
    xf = _f32(x).reshape(48, 8, 128).astype(np.float64)
    s = sf[:, :48].T.astype(np.float64)[:, :, None]
    quo = (xf / s).astype(np.float32)  # fp64 quotient rounded once to fp32
    ref = torch.from_numpy(quo.reshape(48, 1024)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


def test_amax_element_gets_max_code():
    x = bf16_normal((40, 2048), seed=31)
    q, _ = quant.quant_1x128(x)
    xf = np.abs(_f32(x)).reshape(40, 16, 128)
    idx = xf.argmax(axis=2)
    qq = q.reshape(40, 16, 128)
    picked = np.take_along_axis(qq, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all((picked & 0x7F) == 0x7E)


def test_dequantisation_error_bound():
    x = bf16_normal((64, 1024), seed=41)
    q, sf = quant.quant_1x128(x)
    xf = _f32(x).astype(np.float64).reshape(64, 8, 128)
    s = sf[:, :64].T.astype(np.float64)[:, :, None]
    deq = e4m3.decode(q).reshape(64, 8, 128) * s
    err = np.abs(deq - xf)
    # normal e4m3 range: half an ulp is 2^-4 relative; subnormal: 2^-10 absolute
    # (times s); plus the fp32 rounding of the quotient.
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * s) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)
    assert np.all(np.abs(sf[:, :64] * 448.0 - np.abs(xf).max(axis=2).T) <= np.spacing(np.abs(xf).max(axis=2).T.astype(np.float32)))


@pytest.mark.parametrize("j", [-3, 5])
def test_power_of_two_invariance(j):
    x = bf16_normal((16, 512), seed=51)
    q, sf = quant.quant_1x128(x)
    scaled = torch.from_numpy(_f32(x) * np.float32(2.0 ** j)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q2, sf2 = quant.quant_1x128(scaled)
    assert np.array_equal(q, q2)
    assert np.array_equal(sf2, (sf * np.float32(2.0 ** j)).astype(np.float32))


def test_zero_and_negative_zero_tiles():
    x = bf16_normal((4, 384), seed=61)
    x[1, 128:256] = 0x0000
    x[2, 0:128] = 0x8000  # -0.0
    x[3, 256:384] = np.where(np.arange(128) % 2 == 0, 0x8000, 0x0000).astype(np.uint16)
    q, sf = quant.quant_1x128(x)
    assert sf[1, 1] == 0 and np.all(q[1, 128:256] == 0x00)
    assert sf[0, 2] == 0 and np.all(q[2, 0:128] == 0x80)
    assert sf[2, 3] == 0 and np.array_equal(q[3, 256:384], np.where(np.arange(128) % 2 == 0, 0x80, 0x00))
    assert sf[0, 0] > 0


def test_tiny_amax_keeps_subnormal_scale():
    # amax = 2^-120: s = 2^-120/448 is an fp32 subnormal and must not flush.
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 0] = 0x0380  # bf16 2^-120
    x[0, 1] = 0x8300  # bf16 -2^-121
    x[0, 2] = 0x0001  # smallest bf16 subnormal 2^-133
    q, sf = quant.quant_1x128(x)
    s = sf[0, 0]
    assert 0 < s < np.finfo(np.float32).tiny
    assert s == _scale_fp64_route(2.0 ** -120)
    assert q[0, 0] == 0x7E
    quo = np.float32(-(2.0 ** -121) / float(s))
    assert q[0, 1] == torch.tensor([quo]).to(torch.float8_e4m3fn).view(torch.uint8).item()


def test_quotient_above_448_clamps():
    # A tile whose only non-zero is the smallest bf16 subnormal: s = 2^-133/448
    # is a coarse fp32 subnormal, x/s lands above 448 and clamps (satfinite).
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 5] = 0x0001
    q, sf = quant.quant_1x128(x)
    assert float(2.0 ** -133) / float(sf[0, 0]) > 448.0
    assert q[0, 5] == 0x7E


@pytest.mark.parametrize("n,k", [(128, 128), (200, 256), (2112 // 8, 384), (80, 128)])
def test_128x128_layout_and_partial_block(n, k):
    w = bf16_normal((n, k), seed=71 + n)
    q, sf = quant.quant_128x128(w)
    nb = (n + 127) // 128
    assert q.shape == (n, k) and sf.shape == (nb, k // 128)
    wf = _f32(w)
    for i in range(nb):
        for j in range(k // 128):
            blk = wf[i * 128:min(n, (i + 1) * 128), j * 128:(j + 1) * 128]
            assert sf[i, j] == _scale_fp64_route(np.abs(blk).max())
            quo = (blk.astype(np.float64) / float(sf[i, j])).astype(np.float32)
            ref = torch.from_numpy(quo).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[i * 128:min(n, (i + 1) * 128), j * 128:(j + 1) * 128], ref)


def test_partial_block_ignores_rows_past_n():
    # N = 130: the second block has 2 valid rows; its amax must come from them.
    w = bf16_normal((130, 128), seed=81)
    w[128:] = torch.tensor([[0.5] * 128, [-0.25] * 128]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _, sf = quant.quant_128x128(w)
    assert sf[1, 0] == np.float32(0.5 / 448.0)


def test_block_quantisers_agree_on_row_constant_blocks():
    # If every row of a 128x128 block is the same, each 1x128 tile has the
    # block's amax, so both quantisers must produce identical codes and scales.
    row = bf16_normal((1, 256), seed=91)
    w = np.repeat(row, 128, axis=0)
    q1, sf1 = quant.quant_1x128(w)
    q2, sf2 = quant.quant_128x128(w)
    assert np.array_equal(q1, q2)
    assert np.all(sf1[:, :128] == sf2[0][:, None])


def test_grouped_activation_layout():
    x = bf16_normal((3, 10, 256), seed=95)
    q, sf = quant.quant_1x128(x)
    assert q.shape == (3, 10, 256) and sf.shape == (3, 2, 12)
    for g in range(3):
        qg, sfg = quant.quant_1x128(x[g])
        assert np.array_equal(q[g], qg) and np.array_equal(sf[g], sfg)


def test_rejects_non_finite():
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 0] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        quant.quant_1x128(x)
