"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

Nothing in here quantises, multiplies or scales: it only draws random numbers
and builds index arrays, so both the CPU oracle and the HIP path can consume
the same bytes without sharing any of the method's arithmetic.

Recipe (the pages measure DeepSeek-V3/R1 inference shapes but name no input
distribution, so i.i.d. N(0,1) values stand in for activations and weights):
* values: numpy default_rng(seed).standard_normal(shape, float32), then RNE to
  bf16 (torch's CPU cast), stored as uint16 bit patterns;
* seeds: A = 1000 + workload number, B = 2000 + workload number;
* contiguous m_indices: expert g repeated for its (128-aligned) segment;
* masked_m: default_rng(3000).integers(1, M_max + 1, size=G), or M_max for
  every group in the all-valid masked workloads of the pages' tables.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

SEED_A = 1000
SEED_B = 2000
SEED_MASK = 3000


def bf16_normal(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, scale^2) values rounded to bf16, as uint16 bit patterns."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# bf16 patterns of 0, +-0.5, +-1 and +-1.75.
_GRID_BITS = np.array([0x0000, 0x3F00, 0xBF00, 0x3F80, 0xBF80, 0x3FE0, 0xBFE0], dtype=np.uint16)


def bf16_grid(shape, seed: int) -> np.ndarray:
    """Values drawn uniformly from {0, +-0.5, +-1, +-1.75}, with +1.75 placed at
    the first element of every 128-wide slice of the last axis, as uint16 bf16
    patterns.  Every 1x128 tile (and so every 128x128 block) then has amax
    1.75, a value set on which products and sums stay small dyadic numbers."""
    if shape[-1] % 128:
        raise ValueError("last axis must be a multiple of 128")
    rng = np.random.default_rng(seed)
    x = _GRID_BITS[rng.integers(0, _GRID_BITS.size, size=shape)]
    x[..., ::128] = 0x3FE0
    return x


def contiguous_m_indices(segment_rows, pad_rows=None, order=None) -> np.ndarray:
    """Per-row expert ids for the contiguous layout.

    segment_rows[g] rows for expert g, followed by pad_rows[g] rows of -1
    (padding up to the alignment).  `order` permutes the experts' segments.
    """
    groups = len(segment_rows)
    pad_rows = pad_rows or [0] * groups
    order = list(range(groups)) if order is None else list(order)
    parts = []
    for g in order:
        parts.append(np.full(segment_rows[g], g, dtype=np.int32))
        parts.append(np.full(pad_rows[g], -1, dtype=np.int32))
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int32)


def masked_m(groups: int, m_max: int, seed: int = SEED_MASK) -> np.ndarray:
    """Valid-row counts per expert, uniform in [1, m_max]."""
    return np.random.default_rng(seed).integers(1, m_max + 1, size=groups).astype(np.int32)


@dataclass
class Workload:
    """One benchmark workload: layout and sizes, plus its seeds."""

    name: str
    layout: str  # "dense" | "contiguous" | "masked"
    m: int  # rows per group (dense: M; contiguous: rows per expert; masked: M_max)
    n: int
    k: int
    groups: int = 1
    number: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def seed_a(self) -> int:
        return SEED_A + self.number

    @property
    def seed_b(self) -> int:
        return SEED_B + self.number

    @property
    def all_valid(self) -> bool:
        return bool(self.extra.get("all_valid", False))


def workload_masked_m(wl: "Workload") -> np.ndarray:
    """masked_m of a masked workload: seeded random counts, or all rows valid."""
    if wl.all_valid:
        return np.full(wl.groups, wl.m, dtype=np.int32)
    return masked_m(wl.groups, wl.m)


NK_PAIRS = [(2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168), (7168, 2048)]


def workloads():
    """The five workloads of the DeepSeek-V3 shapes this library is measured on."""
    out = [Workload("dense_m64_n2112_k7168", "dense", 64, 2112, 7168, number=1)]
    for n, k in NK_PAIRS:
        out.append(Workload(f"dense_m128_n{n}_k{k}", "dense", 128, n, k, number=2))
    for n, k in NK_PAIRS:
        out.append(Workload(f"dense_m4096_n{n}_k{k}", "dense", 4096, n, k, number=3))
    out.append(Workload("contiguous_g4_m8192_n4096_k7168", "contiguous", 8192, 4096, 7168, groups=4, number=4))
    out.append(Workload("masked_g4_mmax1024_n4096_k7168", "masked", 1024, 4096, 7168, groups=4, number=5))
    return out


def extra_workloads():
    """Shapes beyond the pages' tables: the K-grouped weight-gradient GEMM of
    an 8-expert MoE layer, M = 7168 (hidden) x N = 2048 (expert
    intermediate), 8192 tokens in unequal 128-aligned groups (one empty), and
    the same with equal groups."""
    return [Workload("k_grouped_g8_m7168_n2048_k8192", "k_grouped", 7168, 2048, 8192, groups=8, number=6,
                     extra={"tokens": [1024, 640, 1536, 0, 1152, 2048, 896, 896]}),
            Workload("k_grouped_g8_m7168_n2048_k8192_equal", "k_grouped", 7168, 2048, 8192, groups=8, number=6,
                     extra={"tokens": [1024] * 8})] + majors_workloads()


def majors_workloads():
    """The dense prefill (4096 x 4096 x 7168) and decode (128 x 7168 x 16384)
    shapes in the NN, TN and TT operand majors (A stored [K][M] for T, B
    stored [K][N] for the second letter N).  Same seeds as the NT shapes."""
    out = []
    for mj in ("nn", "tn", "tt"):
        out.append(Workload(f"dense_{mj}_m4096_n4096_k7168", "dense", 4096, 4096, 7168, number=3,
                            extra={"majors": mj}))
        out.append(Workload(f"dense_{mj}_m128_n7168_k16384", "dense", 128, 7168, 16384, number=2,
                            extra={"majors": mj}))
    return out


def k_group_offsets(wl: "Workload") -> np.ndarray:
    """[G + 1] int32 K offsets of a K-grouped workload's token groups."""
    return np.concatenate([[0], np.cumsum(wl.extra["tokens"])]).astype(np.int32)


def pages_workloads():
    """The rows of the pages' performance tables (DeepGEMM project introduction,
    section Performance) not already among workloads(): dense M = 64 at the
    other five (N, K) pairs, contiguous 4 x 8192 at (7168, 2048) and 8 x 4096 at
    both pairs, masked 1 x 1024, 2 x 512 and 4 x 256 with every row valid at
    both pairs.  Seeds follow the workload numbers of workloads()."""
    out = []
    for n, k in NK_PAIRS[1:]:
        out.append(Workload(f"dense_m64_n{n}_k{k}", "dense", 64, n, k, number=1))
    out.append(Workload("contiguous_g4_m8192_n7168_k2048", "contiguous", 8192, 7168, 2048, groups=4, number=4))
    for n, k in [(4096, 7168), (7168, 2048)]:
        out.append(Workload(f"contiguous_g8_m4096_n{n}_k{k}", "contiguous", 4096, n, k, groups=8, number=4))
    for g, mm in [(1, 1024), (2, 512), (4, 256)]:
        for n, k in [(4096, 7168), (7168, 2048)]:
            out.append(Workload(f"masked_g{g}_m{mm}_full_n{n}_k{k}", "masked", mm, n, k, groups=g, number=5,
                                extra={"all_valid": True}))
    return out
