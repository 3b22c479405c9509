"""GPU parity of the GEMMs at sizes the oracle computes in full: every output
element is compared with the oracle's fp64 result under the bf16 tolerance
rule; rows and columns the method must not write are checked against a
sentinel bit for bit; closed-form cases are checked bit for bit."""

import numpy as np
import pytest
import torch

from oracle import e4m3, gemm, quant
from synth import bf16_normal, contiguous_m_indices
from tests.gpu_util import SENTINEL, bf16_to_f64, dev, host, require_gpu
from tests.tolerance import check

pytestmark = pytest.mark.gpu


def _operands(m, n, k, seed, groups=None, a_shape=None):
    xa = bf16_normal(a_shape or (m, k), seed)
    xb = bf16_normal((n, k) if groups is None else (groups, n, k), seed + 1)
    a, sfa = quant.quant_1x128(xa)
    b, sfb = quant.quant_128x128(xb)
    return a, sfa, b, sfb


def _workspace(dg, m, n, k, groups=1):
    size = dg.dg_get_workspace_size(m, n, k, groups)
    return torch.zeros(max(size, 16), dtype=torch.uint8, device="cuda") if size else None


def run_dense(dg, a, sfa, b, sfb, ldd=None):
    m, n = a.shape[0], b.shape[0]
    ldd = ldd or n
    full = torch.full((m, ldd), SENTINEL, dtype=torch.int16, device="cuda")
    d = full[:, :n]
    dg.dg_fp8_gemm_nt(dev(a), dev(sfa), dev(b), dev(sfb), d, workspace=_workspace(dg, m, n, a.shape[1]))
    return host(full)


DENSE_SHAPES = [
    (1, 16, 128), (16, 16, 128), (33, 80, 128), (64, 2112, 7168), (128, 200, 384),
    (130, 136, 256), (257, 384, 512), (96, 1000, 1024), (200, 392, 2048), (512, 512, 256),
]


@pytest.mark.parametrize("m,n,k", DENSE_SHAPES)
def test_dense_matches_oracle(m, n, k):
    dg = require_gpu()
    a, sfa, b, sfb = _operands(m, n, k, seed=1000 + m + n)
    out = run_dense(dg, a, sfa, b, sfb)
    ref = gemm.gemm_nt_ref(a, sfa, b, sfb)
    check(bf16_to_f64(out), ref, f"dense {m}x{n}x{k}")


def test_dense_strided_output_leaves_padding_columns():
    dg = require_gpu()
    m, n, k = 70, 136, 256
    a, sfa, b, sfb = _operands(m, n, k, seed=3)
    out = run_dense(dg, a, sfa, b, sfb, ldd=n + 24)
    assert np.all(out[:, n:] == SENTINEL)
    check(bf16_to_f64(out[:, :n]), gemm.gemm_nt_ref(a, sfa, b, sfb), "strided d")


def test_dense_k_zero_writes_zeros():
    # An empty contraction: every output is the empty sum, +0.
    dg = require_gpu()
    a = torch.zeros((5, 16), dtype=torch.uint8, device="cuda")[:, :0]
    b = torch.zeros((24, 16), dtype=torch.uint8, device="cuda")[:, :0]
    sfa = torch.zeros((1, 8), dtype=torch.float32, device="cuda")[:0]
    sfb = torch.zeros((1, 1), dtype=torch.float32, device="cuda")[:, :0]
    full = torch.full((5, 24), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt(a, sfa, b, sfb, full)
    assert np.all(host(full) == 0)


def test_one_hot_is_bit_exact():
    # D[i][n] = dec(B[n][kk[i]]) * sb (power of two): exact in bf16, so the GPU
    # result must equal it bit for bit.
    dg = require_gpu()
    m, n, k = 64, 392, 1024
    rng = np.random.default_rng(9)
    kk = rng.integers(0, k, m)
    a = np.zeros((m, k), dtype=np.uint8)
    a[np.arange(m), kk] = 0x38
    sfa = np.ones((k // 128, m), dtype=np.float32)
    b, _ = quant.quant_128x128(bf16_normal((n, k), 3))
    sfb = (2.0 ** rng.integers(-8, 8, ((n + 127) // 128, k // 128))).astype(np.float32)
    ref = gemm.gemm_nt_ref(a, sfa, b, sfb)
    out = run_dense(dg, a, sfa, b, sfb)
    assert np.array_equal(bf16_to_f64(out), ref)


def test_power_of_two_scale_invariance_is_bit_exact():
    dg = require_gpu()
    m, n, k = 128, 256, 1024
    a, sfa, b, sfb = _operands(m, n, k, seed=44)
    base = run_dense(dg, a, sfa, b, sfb)
    moved = run_dense(dg, a, sfa * np.float32(16), b, sfb / np.float32(16))
    assert np.array_equal(base, moved)
    doubled = run_dense(dg, a, sfa * np.float32(2), b, sfb)
    assert np.array_equal(bf16_to_f64(doubled), 2 * bf16_to_f64(base))
    flipped = run_dense(dg, a ^ np.uint8(0x80), sfa, b, sfb)
    assert np.array_equal(bf16_to_f64(flipped), -bf16_to_f64(base))


def test_dense_is_deterministic():
    dg = require_gpu()
    a, sfa, b, sfb = _operands(128, 2112, 7168, seed=8)
    first = run_dense(dg, a, sfa, b, sfb)
    for _ in range(3):
        assert np.array_equal(run_dense(dg, a, sfa, b, sfb), first)


# ------------------------------------------------------------ contiguous --

def run_contiguous(dg, a, sfa, b, sfb, mi):
    m_total, n = a.shape[0], b.shape[1]
    d = torch.full((m_total, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_grouped_contiguous(dev(a), dev(sfa), dev(b), dev(sfb), d, dev(mi.astype(np.int32)),
                             workspace=_workspace(dg, m_total, n, a.shape[1], b.shape[0]))
    return host(d)


@pytest.mark.parametrize("sizes,pads,order,n,k", [
    ([128, 256, 384, 128], [0, 0, 0, 0], [0, 1, 2, 3], 256, 512),
    ([100, 200, 0, 30], [28, 56, 128, 98], [3, 1, 0, 2], 136, 384),
    ([384, 128], [0, 0], [1, 0], 2112, 1024),
])
def test_contiguous_matches_oracle(sizes, pads, order, n, k):
    dg = require_gpu()
    groups = len(sizes)
    mi = contiguous_m_indices(sizes, pads, order)
    a, sfa, b, sfb = _operands(mi.size, n, k, seed=70 + n, groups=groups)
    out = run_contiguous(dg, a, sfa, b, sfb, mi)
    ref, written = gemm.grouped_contiguous_ref(a, sfa, b, sfb, mi)
    assert np.all(out[~written] == SENTINEL)
    check(bf16_to_f64(out[written]), ref[written], "contiguous")


def test_contiguous_group_indexing_is_exact():
    dg = require_gpu()
    groups, n, k = 4, 64, 128
    mi = contiguous_m_indices([128, 256, 128, 128], order=[2, 0, 3, 1])
    mi[-5:] = -1
    mi[130] = 7  # out-of-range id: a padding row
    a = np.zeros((mi.size, k), dtype=np.uint8)
    a[:, 0] = 0x38
    sfa = np.ones((1, mi.size), dtype=np.float32)
    b = np.zeros((groups, n, k), dtype=np.uint8)
    for g, c in enumerate([0x38, 0x40, 0x44, 0x48]):
        b[g, :, 0] = c
    sfb = np.ones((groups, 1, 1), dtype=np.float32)
    out = run_contiguous(dg, a, sfa, b, sfb, mi)
    ref, written = gemm.grouped_contiguous_ref(a, sfa, b, sfb, mi)
    assert np.all(out[~written] == SENTINEL)
    assert np.array_equal(bf16_to_f64(out[written]), ref[written])


# ---------------------------------------------------------------- masked --

def run_masked(dg, a, sfa, b, sfb, mm, expected_m=0):
    groups, m_max, n = a.shape[0], a.shape[1], b.shape[1]
    d = torch.full((groups, m_max, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_grouped_masked(dev(a), dev(sfa), dev(b), dev(sfb), d, dev(np.asarray(mm, dtype=np.int32)),
                         expected_m=expected_m, workspace=_workspace(dg, m_max, n, a.shape[2], groups))
    return host(d)


@pytest.mark.parametrize("m_max,mm,n,k", [
    (256, [0, 1, 127, 128], 256, 512),
    (256, [129, 256, 300, -4], 136, 384),
    (200, [200, 7, 64, 65], 2112, 1024),
    (1024, [1024, 513, 2, 1000], 512, 256),
])
def test_masked_matches_oracle_and_leaves_rows(m_max, mm, n, k):
    dg = require_gpu()
    groups = len(mm)
    a, sfa, b, sfb = _operands(None, n, k, seed=90 + m_max, groups=groups, a_shape=(groups, m_max, k))
    out = run_masked(dg, a, sfa, b, sfb, mm, expected_m=int(np.mean(np.clip(mm, 0, m_max))))
    ref, written = gemm.grouped_masked_ref(a, sfa, b, sfb, np.array(mm))
    assert np.all(out[~written] == SENTINEL)
    if written.any():
        check(bf16_to_f64(out[written]), ref[written], "masked")


def test_masked_all_empty_is_noop():
    dg = require_gpu()
    a, sfa, b, sfb = _operands(None, 128, 128, seed=5, groups=2, a_shape=(2, 64, 128))
    out = run_masked(dg, a, sfa, b, sfb, [0, 0])
    assert np.all(out == SENTINEL)


def test_workspace_reused_across_shapes_and_configurations():
    # One workspace, zero-filled once and sized for the largest call, serves a
    # sequence of stream-K GEMMs whose configurations differ (128x128 tiles in
    # 4 parts, 64x64 tiles in 4 parts, the quantised-output form's widened
    # tiles, then the first shape again).  The arrival counters sit at the
    # same place for every configuration and each call leaves them at zero,
    # so every output must match the oracle.
    dg = require_gpu()
    shapes = [(128, 7168, 16384), (128, 4096, 7168), (64, 2112, 7168), (128, 7168, 16384)]
    size = max(dg.dg_get_workspace_size(m, n, k, 1) for m, n, k in shapes)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for i, (m, n, k) in enumerate(shapes):
        a, sfa, b, sfb = _operands(m, n, k, seed=4100 + i)
        full = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
        dg.dg_fp8_gemm_nt(dev(a), dev(sfa), dev(b), dev(sfb), full, workspace=ws)
        rows = np.arange(0, m, 7)
        ref = gemm.gemm_nt_ref(a[rows], sfa[:, rows], b, sfb)
        check(bf16_to_f64(host(full)[rows]), ref, f"reused workspace, call {i}: {m}x{n}x{k}")
    counters = host(ws[: 8192 * 4].view(torch.int32))
    assert not np.any(counters), "arrival counters left non-zero"
