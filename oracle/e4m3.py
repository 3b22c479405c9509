"""OCP e4m3fn (FP8) codec, written from the format definition.

The pages only say "FP8" (DeepGEMM project introduction, opening section;
hbcasj.com news article).  The flavour is read as OCP e4m3fn: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN only at
S.1111.111, largest finite magnitude 448.  The 448 maximum is what the
amax/448 scale rule presumes; gfx950 uses this same flavour natively.

Encoding rule (a reading, the pages give none): round |v| to the nearest of
the 127 finite non-negative e4m3 values, ties to the value whose code is even
(even mantissa), keep the sign bit (so -0 and tiny negatives give 0x80), and
clamp magnitudes above 448 to 448 ("satfinite").  NaN and infinite inputs are
outside the contract and are rejected.
"""

import numpy as np

NAN_CODES = (0x7F, 0xFF)
MAX_FINITE = 448.0


def decode_one(code: int) -> float:
    """Value of one byte under OCP e4m3fn, from its three bit fields."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:  # subnormal: (m/8) * 2^(1-7)
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def decode_table() -> np.ndarray:
    """fp64 value of every code 0..255 (NaN at 0x7F and 0xFF)."""
    return np.array([decode_one(c) for c in range(256)], dtype=np.float64)


_DEC = decode_table()
# The finite non-negative values, in code order 0x00..0x7E; they are
# strictly increasing in the code, which the encoder relies on.
_POS = _DEC[:0x7F].copy()


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode a uint8 array to exact fp64 values."""
    return _DEC[np.asarray(codes, dtype=np.uint8)]


def encode_rne(v) -> np.ndarray:
    """Encode fp32 values to e4m3fn codes: nearest, ties to even, satfinite."""
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3 encoder: NaN/Inf input is outside the contract")
    neg = np.signbit(v)
    a = np.abs(v).astype(np.float64)  # exact widening
    a = np.minimum(a, MAX_FINITE)  # satfinite clamp
    hi = np.searchsorted(_POS, a, side="left")  # _POS[hi-1] < a <= _POS[hi]
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]  # exact: operands are within 53 bits of each other
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS[hi], hi, code)  # exact hits (includes 0)
    return (code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)
