"""K-axis grouped GEMM (the weight-gradient shape of MoE training).

Test infrastructure only (see oracle/__init__.py).

What the pages fix: besides grouping along M, the library groups along the K
axis for MoE ("DeepGEMM: efficient BLAS kernel library on GPU", yfxerp.com,
section 3.2: grouped GEMM along the M or the K axis).  They say nothing more.
Reading taken here (the plainest one consistent with the rest):

* the tokens of all experts are concatenated along K, expert g owning the
  128-aligned range [k_offsets[g], k_offsets[g+1]);
* both operands are activation-like (e.g. output gradients and layer inputs
  of the expert's tokens), so both carry the activation quantiser's 1x128
  scales along K: sfa [K/128][ld_a] per row of A, sfb [K/128][ld_b] per row
  of B (the "1D-1D" scaling, produced by the 1x128 quantiser for each);
* D_g[m][n] = sum over the slices kb of group g of
      P_kb[m][n] * (sfa[kb][m] * sfb[kb][n]),
  P_kb the exact partial product of the slice, promoted per 128-K slice as
  in the M-grouped GEMMs; an empty group gives D_g = 0.

Computed here exactly per slice in fp64 (as in gemm.py).
"""

from fractions import Fraction

import numpy as np

from . import e4m3

BLOCK = 128


def _ranges(k_offsets, k_total):
    offs = [int(x) for x in k_offsets]
    if offs[0] != 0 or offs[-1] != k_total or any(b < a for a, b in zip(offs, offs[1:])):
        raise ValueError("k_offsets must start at 0, end at K and not decrease")
    if any(x % BLOCK for x in offs):
        raise ValueError("group boundaries must be multiples of 128")
    return [(a // BLOCK, b // BLOCK) for a, b in zip(offs, offs[1:])]


def k_grouped_ref(a_q, sfa, b_q, sfb, k_offsets) -> np.ndarray:
    """a_q [M][K], sfa [K/128][ld >= M], b_q [N][K], sfb [K/128][ld >= N],
    k_offsets [G+1] -> D64 [G][M][N]."""
    a_q = np.asarray(a_q, dtype=np.uint8)
    b_q = np.asarray(b_q, dtype=np.uint8)
    sfa = np.asarray(sfa, dtype=np.float32)
    sfb = np.asarray(sfb, dtype=np.float32)
    m, k = a_q.shape
    n = b_q.shape[0]
    if b_q.shape[1] != k or k % BLOCK:
        raise ValueError("A and B must share K, a multiple of 128")
    if sfa.shape[0] != k // BLOCK or sfa.shape[1] < m or sfb.shape[0] != k // BLOCK or sfb.shape[1] < n:
        raise ValueError("scales must be [K/128][ld >= rows] for both operands")
    a = e4m3.decode(a_q)
    b = e4m3.decode(b_q)
    ranges = _ranges(k_offsets, k)
    d = np.zeros((len(ranges), m, n), dtype=np.float64)
    for g, (kb0, kb1) in enumerate(ranges):
        for kb in range(kb0, kb1):
            sl = slice(kb * BLOCK, (kb + 1) * BLOCK)
            partial = a[:, sl] @ b[:, sl].T  # exact in fp64
            scale = sfa[kb, :m].astype(np.float64)[:, None] * sfb[kb, :n].astype(np.float64)[None, :]
            d[g] += partial * scale
    return d


def k_grouped_brute(a_q, sfa, b_q, sfb, k_offsets):
    """Exact rational D_g (nested lists of Fraction) by plain loops; tiny shapes only."""
    a_q = np.asarray(a_q, dtype=np.uint8)
    b_q = np.asarray(b_q, dtype=np.uint8)
    m, k = a_q.shape
    n = b_q.shape[0]
    dec = [None if c in e4m3.NAN_CODES else Fraction(e4m3.decode_one(c)) for c in range(256)]
    out = []
    for kb0, kb1 in _ranges(k_offsets, k):
        dg = []
        for i in range(m):
            row = []
            for j in range(n):
                total = Fraction(0)
                for kb in range(kb0, kb1):
                    part = sum((dec[int(a_q[i, kk])] * dec[int(b_q[j, kk])]
                                for kk in range(kb * BLOCK, (kb + 1) * BLOCK)), Fraction(0))
                    total += part * Fraction(float(sfa[kb][i])) * Fraction(float(sfb[kb][j]))
                row.append(total)
            dg.append(row)
        out.append(dg)
    return out
