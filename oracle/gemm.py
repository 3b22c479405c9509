"""Reference GEMMs with fine-grained scaling: D = A . B^T, bf16 output.

The method ("DeepGEMM project introduction", section Interfaces; "Deepseek
DeepGEMM technical principles", section "Technical background and core
principles"): A is [M][K] e4m3 with one fp32 scale per row and 128-wide K
slice, B is [N][K] e4m3 (the NT layout: both operands K-contiguous) with one
fp32 scale per 128x128 block.  Each 128-wide K slice is a low-precision
partial product; it is scaled by sa*sb and promoted into a higher-precision
accumulator (promotion interval N_C = 128).

Here each partial product is computed in fp64, where it is exact: an e4m3
product is a multiple of 2^-18 below 2^18, so a sum of 128 of them needs at
most 43 significant bits.  The scale product sa*sb (two fp32 values) is exact
in fp64 as well; only the promotion multiply and add round, at fp64.  The
result D64 is therefore within about K/128 * 2^-53 (relative) of the exact
value, and is the reference the bf16 output is compared against.

Grouped layouts (same sections of the project introduction):
* contiguous: tokens of all experts are concatenated along M, each expert's
  segment aligned to 128 rows; m_indices[r] names the expert of row r.
  Reading: rows whose index is < 0 or >= G (padding) are not written.
* masked: A is [G][M_max][K]; masked_m[g] rows of group g are valid, the
  rest are not written.  Reading: masked_m is clamped to [0, M_max].
"""

from fractions import Fraction

import numpy as np

from . import e4m3

BLOCK = 128


def _check(a_q, sfa, b_q, sfb):
    m, k = a_q.shape
    n, kb_ = b_q.shape
    if kb_ != k or k % BLOCK:
        raise ValueError("A and B must share K, a multiple of 128")
    if sfa.shape[0] != k // BLOCK or sfa.shape[1] < m:
        raise ValueError("sfa must be [K/128][ld >= M]")
    if sfb.shape != ((n + BLOCK - 1) // BLOCK, k // BLOCK):
        raise ValueError("sfb must be [ceil(N/128)][K/128]")


def gemm_nt_ref(a_q, sfa, b_q, sfb) -> np.ndarray:
    """Dense NT GEMM: D64[m][n] = sum_kb P_kb[m][n] * (sa[kb][m] * sb[n/128][kb])."""
    a_q = np.asarray(a_q, dtype=np.uint8)
    b_q = np.asarray(b_q, dtype=np.uint8)
    sfa = np.asarray(sfa, dtype=np.float32)
    sfb = np.asarray(sfb, dtype=np.float32)
    _check(a_q, sfa, b_q, sfb)
    m, k = a_q.shape
    n = b_q.shape[0]
    a = e4m3.decode(a_q)
    b = e4m3.decode(b_q)
    col_block = np.arange(n) // BLOCK
    d = np.zeros((m, n), dtype=np.float64)
    for kb in range(k // BLOCK):
        sl = slice(kb * BLOCK, (kb + 1) * BLOCK)
        partial = a[:, sl] @ b[:, sl].T  # exact in fp64
        scale = sfa[kb, :m].astype(np.float64)[:, None] * sfb[col_block, kb].astype(np.float64)[None, :]
        d += partial * scale
    return d


def grouped_contiguous_ref(a_q, sfa, b_q, sfb, m_indices):
    """Contiguous grouped GEMM.

    a_q [M_total][K], sfa [K/128][ld >= M_total], b_q [G][N][K],
    sfb [G][ceil(N/128)][K/128], m_indices int [M_total].
    Returns (D64 [M_total][N] with NaN on unwritten rows, written bool [M_total]).
    """
    a_q = np.asarray(a_q, dtype=np.uint8)
    m_indices = np.asarray(m_indices, dtype=np.int64)
    groups, n = b_q.shape[0], b_q.shape[1]
    m_total = a_q.shape[0]
    d = np.full((m_total, n), np.nan, dtype=np.float64)
    written = (m_indices >= 0) & (m_indices < groups)
    for g in range(groups):
        rows = np.nonzero(m_indices == g)[0]
        if rows.size == 0:
            continue
        d[rows] = gemm_nt_ref(a_q[rows], np.asarray(sfa)[:, rows], b_q[g], sfb[g])
    return d, written


def grouped_masked_ref(a_q, sfa, b_q, sfb, masked_m):
    """Masked grouped GEMM.

    a_q [G][M_max][K], sfa [G][K/128][ld >= M_max], b_q [G][N][K],
    sfb [G][ceil(N/128)][K/128], masked_m int [G].
    Returns (D64 [G][M_max][N] with NaN on unwritten rows, written bool [G][M_max]).
    """
    a_q = np.asarray(a_q, dtype=np.uint8)
    groups, m_max, _ = a_q.shape
    n = b_q.shape[1]
    d = np.full((groups, m_max, n), np.nan, dtype=np.float64)
    written = np.zeros((groups, m_max), dtype=bool)
    for g in range(groups):
        mm = int(min(max(int(masked_m[g]), 0), m_max))
        if mm == 0:
            continue
        d[g, :mm] = gemm_nt_ref(a_q[g, :mm], np.asarray(sfa)[g][:, :mm], b_q[g], sfb[g])
        written[g, :mm] = True
    return d, written


def brute_force_exact(a_q, sfa, b_q, sfb):
    """Exact rational D (list of lists of Fraction), by plain triple loop.

    For tiny shapes only: every code and scale is converted to an exact
    Fraction, so nothing in here rounds.
    """
    a_q = np.asarray(a_q, dtype=np.uint8)
    b_q = np.asarray(b_q, dtype=np.uint8)
    m, k = a_q.shape
    n = b_q.shape[0]
    dec = [None if c in e4m3.NAN_CODES else Fraction(e4m3.decode_one(c)) for c in range(256)]
    out = []
    for i in range(m):
        row = []
        for j in range(n):
            total = Fraction(0)
            for kb in range(k // BLOCK):
                part = Fraction(0)
                for kk in range(kb * BLOCK, (kb + 1) * BLOCK):
                    part += dec[int(a_q[i, kk])] * dec[int(b_q[j, kk])]
                total += part * Fraction(float(sfa[kb][i])) * Fraction(float(sfb[j // BLOCK][kb]))
            row.append(total)
        out.append(row)
    return out
