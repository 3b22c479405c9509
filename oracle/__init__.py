"""CPU oracle for the fine-grained-scaled FP8 GEMM (test infrastructure only).

This package is the slow, obviously correct CPU definition of what the HIP
library computes.  It exists to check the GPU path and nothing else: only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it.  The product path never routes through it, and it shares no code, table or
constant generator with the HIP sources.

Contents
--------
e4m3      OCP e4m3fn decode table and round-to-nearest-even encoder.
quant     1x128 activation and 128x128 weight quantisers (amax/448 scales).
ue8m0     the same quantisers with power-of-two (UE8M0) scales: the smallest
          power of two not below amax/448.
gemm      dense NT, grouped-contiguous and grouped-masked reference GEMMs that
          accumulate each 128-wide K slice exactly in fp64, scale it by
          sa*sb and promote it; plus an exact-rational brute force.
majors    the dense GEMM with the NN, TN and TT operand majors and the 1x128
          quantiser of an M-major (column-stored) activation matrix.
kgrouped  the K-axis grouped GEMM (groups of 128-aligned K ranges, 1x128
          scales along K on both operands) and its exact brute force.
bf16      bit-level helpers for bf16 storage and RNE rounding to bf16.

Sources (the method is described on public pages about DeepSeek's DeepGEMM):
* "DeepGEMM project introduction and local deployment guide"
  (docs.beyondata.com), sections Interfaces, Grouped GEMM (contiguous layout),
  Grouped GEMM (masked layout), Utility functions.
* "Deepseek DeepGEMM technical principles" (blog.51cto.com), section
  "Technical background and core principles": 1x128 activation tiles,
  128x128 weight blocks, promotion every N_C = 128 elements of K.
* "DeepGEMM: efficient BLAS kernel library on GPU" (yfxerp.com), section 3.1:
  scale factors are FP32 on SM90, packed UE8M0 on SM100.

Readings where the pages are silent (e4m3 flavour, the amax/448 scale
formula, the x/s quotient, all-zero tiles, saturation, the -1 convention for
contiguous padding, masked_m clamping) are listed in the module docstrings
that use them.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_*.py against things other than itself (torch's CPU e4m3
cast, exact rational brute force, closed forms, invariants).
"""

from . import bf16, e4m3, gemm, kgrouped, majors, quant, ue8m0  # noqa: F401
