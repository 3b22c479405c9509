"""Power-of-two (UE8M0) scale variant of the two quantisers.

Test infrastructure only (see oracle/__init__.py).

What the pages fix: on their newer architecture the scale factors are UE8M0
(an unsigned 8-bit exponent) packed four to a 32-bit word, instead of fp32
(yfxerp.com DeepGEMM article, section 3.1).  They do not say how such a
scale is chosen.  Reading taken here, the plainest one consistent with the
fp32 rule amax/448: the scale of a tile is the smallest power of two not
below amax/448, so every |x|/s stays within the e4m3 range:

* E = ceil(log2(amax / 448)) + 127 (exactly, on the rational amax/448),
  clamped to [0, 254]; an all-zero tile gets E = 0;
* s = 2^(E - 127);
* q = e4m3_rne(fp32(x / s)): x / s is x times a power of two, so the fp32
  rounding only acts below the fp32 normal range.

Layouts (our choice, four consecutive M or N entries of one K block in one
32-bit word, as the pages pack four UE8M0 per int):
* activations: sf[K/128][ld] uint8 (MN-major), ld = round_up(R, 4), pads 0;
* weights: sf[G][K/128][ld_n] uint8 (MN-major, unlike the fp32 weight
  scales), ld_n = round_up(ceil(N/128), 4), pads 0.
"""

from fractions import Fraction

import numpy as np

from . import bf16, e4m3

BLOCK = 128
ALIGN = 4


def exponent(amax: float) -> int:
    """E of the smallest power of two 2^(E-127) >= amax/448, clamped to [0, 254]."""
    if amax == 0:
        return 0
    r = Fraction(float(amax)) / 448
    k = r.numerator.bit_length() - r.denominator.bit_length()
    while Fraction(2) ** k < r:
        k += 1
    while Fraction(2) ** (k - 1) >= r:
        k -= 1
    return int(min(254, max(0, k + 127)))


def scale_of(e) -> np.ndarray:
    """2^(E-127) as fp64 (exact; also exactly representable in fp32)."""
    return np.ldexp(1.0, np.asarray(e, dtype=np.int64) - 127)


def _codes(x_f32: np.ndarray, e: int) -> np.ndarray:
    quo = np.ldexp(x_f32.astype(np.float64), 127 - e).astype(np.float32)  # exact, then fp32 RN
    return e4m3.encode_rne(quo)


def quant_1x128_ue8m0(x_bits, ld_sf=None):
    """bf16 activations [R][C] (or [G][R][C]) -> (q uint8, sf uint8 [(G)][C/128][ld])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim == 3:
        outs = [quant_1x128_ue8m0(x_bits[g], ld_sf) for g in range(x_bits.shape[0])]
        return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
    rows, cols = x_bits.shape
    if cols % BLOCK:
        raise ValueError("columns must be a multiple of 128")
    ld = (rows + ALIGN - 1) // ALIGN * ALIGN if ld_sf is None else ld_sf
    if ld < rows:
        raise ValueError("scale leading dimension smaller than rows")
    x = bf16.to_f32(x_bits)
    if not np.all(np.isfinite(x)):
        raise ValueError("NaN/Inf input is outside the contract")
    q = np.empty((rows, cols), dtype=np.uint8)
    sf = np.zeros((cols // BLOCK, ld), dtype=np.uint8)
    for r in range(rows):
        for j in range(cols // BLOCK):
            tile = x[r, j * BLOCK:(j + 1) * BLOCK]
            e = exponent(float(np.abs(tile).max()))
            sf[j, r] = e
            q[r, j * BLOCK:(j + 1) * BLOCK] = _codes(tile, e)
    return q, sf


def quant_128x128_ue8m0(w_bits):
    """bf16 weights [N][K] (or [G][N][K]) -> (q uint8, sf uint8 [(G)][K/128][ld_n])."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim == 3:
        outs = [quant_128x128_ue8m0(w_bits[g]) for g in range(w_bits.shape[0])]
        return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
    n, k = w_bits.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    w = bf16.to_f32(w_bits)
    if not np.all(np.isfinite(w)):
        raise ValueError("NaN/Inf input is outside the contract")
    nb, kb = (n + BLOCK - 1) // BLOCK, k // BLOCK
    ld_n = (nb + ALIGN - 1) // ALIGN * ALIGN
    q = np.empty((n, k), dtype=np.uint8)
    sf = np.zeros((kb, ld_n), dtype=np.uint8)
    for i in range(nb):
        r0, r1 = i * BLOCK, min(n, (i + 1) * BLOCK)
        for j in range(kb):
            blk = w[r0:r1, j * BLOCK:(j + 1) * BLOCK]
            e = exponent(float(np.abs(blk).max()))
            sf[j, i] = e
            q[r0:r1, j * BLOCK:(j + 1) * BLOCK] = _codes(blk, e)
    return q, sf


def sfa_as_fp32(sf_u8):
    """Activation exponents -> the fp32 scale layout gemm.py consumes (same shape)."""
    return scale_of(sf_u8).astype(np.float32)


def sfb_as_fp32(sf_u8, n):
    """Weight exponents [(G)][K/128][ld_n] -> fp32 scales [(G)][ceil(N/128)][K/128]."""
    nb = (n + BLOCK - 1) // BLOCK
    s = scale_of(sf_u8).astype(np.float32)
    return np.ascontiguousarray(np.swapaxes(s[..., :nb], -1, -2))
