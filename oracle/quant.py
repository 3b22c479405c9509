"""Fine-grained FP8 quantisers: 1x128 activation tiles, 128x128 weight blocks.

What the pages fix: activations carry one scale per 1x128 tile and weights
one per 128x128 block ("Deepseek DeepGEMM technical principles", section
"Technical background and core principles"); the scales are FP32 (yfxerp.com
article, section 3.1); the activation (LHS) scales are stored transposed,
MN-major, with a padded leading dimension ("DeepGEMM project introduction",
section Interfaces, and the get_tma_aligned_size / get_col_major_tma_aligned_
tensor utilities in section Utility functions).  Casting itself is left to the
caller there; this library ships it as a kernel, so its arithmetic is fixed
here by reading:

* the tile values are the bf16 inputs widened exactly to fp32;
* amax = max |x| over the tile (over the valid rows only for a partial last
  weight block when N is not a multiple of 128);
* s = fp32(amax / 448), one IEEE fp32 division rounded to nearest even;
* q = e4m3_rne(fp32(x / s)), an IEEE fp32 quotient, then the e4m3 encoder
  (this double rounding is part of the definition);
* an all-zero tile gets s = 0 and signed-zero codes (0/0 is read as 0);
* fp32 subnormals are kept throughout (no flush to zero).

Activation scale layout: sf[C/128][ld] with ld = round_up(R, 4) (16-byte
aligned columns); pad entries are 0.  Weight scale layout:
sf[G][ceil(N/128)][K/128].
"""

import numpy as np

from . import bf16, e4m3

BLOCK = 128
SF_ALIGN = 4  # fp32 elements per 16 bytes


def sf_leading_dim(rows: int) -> int:
    """Leading dimension of the transposed activation scale matrix."""
    return (rows + SF_ALIGN - 1) // SF_ALIGN * SF_ALIGN


def _scale(amax: np.ndarray) -> np.ndarray:
    return (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)


def _codes(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Codes of fp32 values x sharing (broadcast) fp32 scale s."""
    zero_tile = s == 0
    safe = np.where(zero_tile, np.float32(1.0), s).astype(np.float32)
    quo = (x / safe).astype(np.float32)
    # amax == 0 means every element is +0 or -0: keep the sign, code 0x00/0x80
    quo = np.where(zero_tile, x, quo).astype(np.float32)
    return e4m3.encode_rne(quo)


def quant_1x128(x_bits, ld_sf=None):
    """Quantise bf16 activations [R][C] (or [G][R][C]) per 1x128 tile.

    Returns (q uint8 same shape, sf float32 [C/128][ld] or [G][C/128][ld]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim == 3:
        outs = [quant_1x128(x_bits[g], ld_sf) for g in range(x_bits.shape[0])]
        return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
    rows, cols = x_bits.shape
    if cols % BLOCK:
        raise ValueError("columns must be a multiple of 128")
    ld = sf_leading_dim(rows) if ld_sf is None else ld_sf
    if ld < rows:
        raise ValueError("scale leading dimension smaller than rows")
    x = bf16.to_f32(x_bits)
    if not np.all(np.isfinite(x)):
        raise ValueError("NaN/Inf input is outside the contract")
    tiles = x.reshape(rows, cols // BLOCK, BLOCK)
    amax = np.abs(tiles).max(axis=2)  # [R][C/128]
    s = _scale(amax)
    q = _codes(tiles, s[:, :, None]).reshape(rows, cols)
    sf = np.zeros((cols // BLOCK, ld), dtype=np.float32)
    sf[:, :rows] = s.T
    return q, sf


def quant_128x128(w_bits):
    """Quantise bf16 weights [N][K] (or [G][N][K]) per 128x128 block.

    Returns (q uint8 same shape, sf float32 [G][ceil(N/128)][K/128]; the G axis
    is present only for 3-D input).
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim == 3:
        outs = [quant_128x128(w_bits[g]) for g in range(w_bits.shape[0])]
        return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
    n, k = w_bits.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    w = bf16.to_f32(w_bits)
    if not np.all(np.isfinite(w)):
        raise ValueError("NaN/Inf input is outside the contract")
    nb, kb = (n + BLOCK - 1) // BLOCK, k // BLOCK
    q = np.empty((n, k), dtype=np.uint8)
    sf = np.empty((nb, kb), dtype=np.float32)
    for i in range(nb):
        r0, r1 = i * BLOCK, min(n, (i + 1) * BLOCK)
        for j in range(kb):
            blk = w[r0:r1, j * BLOCK:(j + 1) * BLOCK]
            s = _scale(np.abs(blk).max())
            sf[i, j] = s
            q[r0:r1, j * BLOCK:(j + 1) * BLOCK] = _codes(blk, s)
    return q, sf
