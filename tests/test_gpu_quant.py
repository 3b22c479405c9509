"""GPU parity of the quantisers: fp8 codes and fp32 scales must equal the
oracle's bit for bit (including the zero padding of the scale matrix)."""

import numpy as np
import pytest
import torch

from oracle import quant
from synth import bf16_normal
from tests.gpu_util import gpu_quant_128x128, gpu_quant_1x128, host, require_gpu

pytestmark = pytest.mark.gpu


def _same_f32(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(1, 128), (5, 256), (33, 384), (64, 7168), (130, 1536), (1000, 512)])
def test_quant_1x128_bit_exact(rows, cols):
    dg = require_gpu()
    x = bf16_normal((rows, cols), seed=500 + rows)
    q, sf = gpu_quant_1x128(dg, x)
    rq, rsf = quant.quant_1x128(x)
    assert np.array_equal(host(q), rq)
    assert _same_f32(host(sf), rsf)


# Heights around the quantiser's rows-per-trip thresholds (one row per trip
# below 2048 rows, two from 2048, four from 16384), with ragged last trips,
# and a grouped matrix whose group boundaries fall inside a four-row trip.
@pytest.mark.parametrize("shape", [(2047, 256), (2051, 384), (16383, 128), (16395, 256), (3, 5467, 128)])
def test_quant_1x128_tall_bit_exact(shape):
    dg = require_gpu()
    x = bf16_normal(shape, seed=510 + shape[-2])
    ld = 5480 if len(shape) == 3 else None
    q, sf = gpu_quant_1x128(dg, x, ld=ld)
    rq, rsf = quant.quant_1x128(x, ld_sf=ld) if ld else quant.quant_1x128(x)
    assert np.array_equal(host(q), rq)
    assert _same_f32(host(sf), rsf)


def test_quant_1x128_grouped_and_wide_ld():
    dg = require_gpu()
    x = bf16_normal((3, 37, 256), seed=77)
    q, sf = gpu_quant_1x128(dg, x, ld=48)
    rq, rsf = quant.quant_1x128(x, ld_sf=48)
    assert np.array_equal(host(q), rq)
    assert _same_f32(host(sf), rsf)


def _special_tiles():
    x = bf16_normal((6, 512), seed=88)
    x[0, 0:128] = 0x0000                      # all +0
    x[1, 128:256] = 0x8000                    # all -0
    x[2, 256:384] = 0
    x[2, 256] = 0x0380                        # amax 2^-120: subnormal fp32 scale
    x[2, 300] = 0x8300
    x[3, 0:128] = 0
    x[3, 5] = 0x0001                          # smallest bf16 subnormal: x/s > 448, clamps
    x[4, 384:512] = np.arange(128, dtype=np.uint16) | 0x0001  # tiny subnormal ramp
    x[5, 0:128] = 0x43E0                      # 448.0 everywhere: s = 1
    return x


def test_quant_1x128_special_tiles():
    dg = require_gpu()
    x = _special_tiles()
    q, sf = gpu_quant_1x128(dg, x)
    rq, rsf = quant.quant_1x128(x)
    assert np.array_equal(host(q), rq)
    assert _same_f32(host(sf), rsf)


def test_quant_encoder_exhaustive_over_bf16():
    # Tiles whose amax is exactly 448 get s = 1, so every other bf16 value in
    # [-448, 448] is encoded as itself: this walks the e4m3 encoder over every
    # bf16 input, including every exact e4m3 midpoint and the subnormals.
    dg = require_gpu()
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = (allbits.astype(np.uint32) << 16).view(np.float32)
    keep = allbits[np.isfinite(vals) & (np.abs(vals) <= 448.0)]
    per = 127
    tiles = ((keep.size + per - 1) // per + 3) // 4 * 4
    padded = np.zeros(tiles * per, dtype=np.uint16)
    padded[:keep.size] = keep
    x = np.concatenate([np.full((tiles, 1), 0x43E0, dtype=np.uint16), padded.reshape(tiles, per)], axis=1)
    x = x.reshape(-1, 512)
    q, sf = gpu_quant_1x128(dg, x)
    rq, rsf = quant.quant_1x128(x)
    assert np.all(rsf[:, :x.shape[0]] == 1.0)
    assert np.array_equal(host(q), rq)
    assert _same_f32(host(sf), rsf)


@pytest.mark.parametrize("shape", [(128, 128), (200, 256), (80, 384), (3, 136, 512), (2112, 1024)])
def test_quant_128x128_bit_exact(shape):
    dg = require_gpu()
    w = bf16_normal(shape, seed=600 + shape[0])
    q, sf = gpu_quant_128x128(dg, w)
    rq, rsf = quant.quant_128x128(w)
    assert np.array_equal(host(q), rq)
    assert _same_f32(host(sf), rsf)


def test_quant_128x128_special_blocks():
    dg = require_gpu()
    w = bf16_normal((130, 256), seed=99)
    w[0:128, 0:128] = 0x8000
    w[128:130, 128:256] = 0
    w[129, 200] = 0x0001
    q, sf = gpu_quant_128x128(dg, w)
    rq, rsf = quant.quant_128x128(w)
    assert np.array_equal(host(q), rq)
    assert _same_f32(host(sf), rsf)


def test_quant_is_deterministic():
    dg = require_gpu()
    x = bf16_normal((256, 1024), seed=5)
    q1, s1 = gpu_quant_1x128(dg, x)
    q2, s2 = gpu_quant_1x128(dg, x)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
