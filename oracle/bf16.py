"""bf16 storage helpers for the oracle.

bf16 values travel as their 16-bit patterns (uint16): the upper half of an
IEEE binary32.  Widening is exact; narrowing from fp64 rounds once to the
nearest bf16 with ties to even (the usual reading of a bf16 output; the pages
only fix the output type, in the API name gemm_fp8_fp8_bf16_nt of the
DeepGEMM project introduction, section Interfaces).
"""

import numpy as np


def to_f32(bits) -> np.ndarray:
    """Exact fp32 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def round_f64(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), kept as fp64.

    bf16 has 8 significant bits and the fp32 exponent range; below 2^-126 the
    spacing stays 2^-133 (subnormals).  Scaling by a power of two is exact, and
    numpy's round() is round-half-to-even.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding: non-finite input")
    _, e = np.frexp(x)  # x = f * 2^e with 0.5 <= |f| < 1
    ulp_exp = np.maximum(e - 8, -133)
    return np.ldexp(np.round(np.ldexp(x, -ulp_exp)), ulp_exp)


def bits_from_f64(x) -> np.ndarray:
    """bf16 bit patterns of fp64 values after RNE rounding to bf16."""
    r = round_f64(x).astype(np.float32)  # exact: r is bf16-representable
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
