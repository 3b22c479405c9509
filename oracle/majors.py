"""The dense GEMM with the other operand majors (NN, TN, TT) and the 1x128
quantiser of an M-major activation matrix.

Source: "DeepGEMM: efficient BLAS kernel library on GPU" (yfxerp.com),
section 3.1, lists NT, TN, NN and TT as the layouts supported from SM100 on,
beside the NT layout of the SM90 kernels, and says no more.  Reading taken
here: the two letters name the operations in D = op(A) . op(B) on row-major
storage, NT being D = A . B^T with a [M][K] and b [N][K] (the NT layout of
gemm.py).  So the stored arrays are

    NT: a [M][K], b [N][K]      NN: a [M][K], b [K][N]
    TT: a [K][M], b [N][K]      TN: a [K][M], b [K][N]

and the result is the NT GEMM of the logical operands A [M][K], B [N][K].
The scales belong to the logical operands and keep the NT layouts:
sfa [K/128][ld] (one per row of A and 128-deep K slice), sfb
[ceil(N/128)][K/128] (one per 128x128 block of B).

An M-major A is quantised along K, i.e. down its columns: quant_1x128_mn
takes x stored [K][M] and forms one scale per column segment of 128 rows,
the 1x128 activation quantiser (quant.py) applied to the logical operand;
quant_1x128_mn_ue8m0 does the same with the power-of-two scales of ue8m0.py.
"""

import numpy as np

from . import bf16, gemm, ue8m0
from .quant import BLOCK, _codes, _scale, sf_leading_dim

LAYOUTS = ("nt", "nn", "tn", "tt")


def logical_operands(layout, a_stored, b_stored):
    """The logical A [M][K] and B [N][K] of stored operands in `layout`."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {LAYOUTS}")
    a_stored = np.asarray(a_stored)
    b_stored = np.asarray(b_stored)
    a = a_stored if layout[0] == "n" else a_stored.T  # 't': stored [K][M]
    b = b_stored if layout[1] == "t" else b_stored.T  # 'n': stored [K][N]
    return np.ascontiguousarray(a), np.ascontiguousarray(b)


def gemm_layout_ref(layout, a_stored, sfa, b_stored, sfb) -> np.ndarray:
    """D64 [M][N] of the dense GEMM in `layout` (see the module docstring)."""
    a, b = logical_operands(layout, a_stored, b_stored)
    return gemm.gemm_nt_ref(a, sfa, b, sfb)


def quant_1x128_mn(x_bits, ld_sf=None):
    """Quantise bf16 x stored [K][M] per 1x128 tile along K (a column segment
    of 128 rows).  Returns (q uint8 [K][M], sf float32 [K/128][ld])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape  # rows = K, cols = M
    if rows % BLOCK:
        raise ValueError("rows (K) must be a multiple of 128")
    ld = sf_leading_dim(cols) if ld_sf is None else ld_sf
    if ld < cols:
        raise ValueError("scale leading dimension smaller than the columns")
    x = bf16.to_f32(x_bits)
    if not np.all(np.isfinite(x)):
        raise ValueError("NaN/Inf input is outside the contract")
    q = np.zeros((rows, cols), dtype=np.uint8)
    sf = np.zeros((rows // BLOCK, ld), dtype=np.float32)
    for kb in range(rows // BLOCK):
        seg = x[kb * BLOCK:(kb + 1) * BLOCK, :]  # [128][M]: column c is tile (kb, c)
        s = _scale(np.abs(seg).max(axis=0))     # [M]
        q[kb * BLOCK:(kb + 1) * BLOCK, :] = _codes(seg, s[None, :])
        sf[kb, :cols] = s
    return q, sf


def quant_1x128_mn_ue8m0(x_bits, ld_sf=None):
    """The column quantiser with UE8M0 scales: (q uint8 [K][M], sf uint8
    [K/128][ld]) with E per column segment as ue8m0.exponent defines it."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    if rows % BLOCK:
        raise ValueError("rows (K) must be a multiple of 128")
    ld = sf_leading_dim(cols) if ld_sf is None else ld_sf
    if ld < cols:
        raise ValueError("scale leading dimension smaller than the columns")
    x = bf16.to_f32(x_bits)
    if not np.all(np.isfinite(x)):
        raise ValueError("NaN/Inf input is outside the contract")
    q = np.zeros((rows, cols), dtype=np.uint8)
    sf = np.zeros((rows // BLOCK, ld), dtype=np.uint8)
    for kb in range(rows // BLOCK):
        for c in range(cols):
            seg = x[kb * BLOCK:(kb + 1) * BLOCK, c]
            e = ue8m0.exponent(float(np.abs(seg).max()))
            sf[kb, c] = e
            q[kb * BLOCK:(kb + 1) * BLOCK, c] = ue8m0._codes(seg, e)
    return q, sf
