"""Pins for the oracle's dense and grouped GEMMs (CPU only).

Checked against: an exact rational brute force on tiny shapes (including a
partial last 128-row weight block and several K slices), fp64 matmul of the
decoded operands when all scales are 1, closed forms for one-hot operands,
sign and power-of-two scale symmetries, grouped = per-group dense, and a
gross-sanity comparison with the unquantised product.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, gemm, quant
from synth import bf16_normal, contiguous_m_indices
from tests.tolerance import check


def _operands(m, n, k, seed):
    a, sfa = quant.quant_1x128(bf16_normal((m, k), seed))
    b, sfb = quant.quant_128x128(bf16_normal((n, k), seed + 1))
    return a, sfa, b, sfb


@pytest.mark.parametrize("m,n,k", [(1, 20, 384), (3, 136, 256), (2, 7, 128)])
def test_matches_exact_brute_force(m, n, k):
    a, sfa, b, sfb = _operands(m, n, k, seed=100 + m)
    d = gemm.gemm_nt_ref(a, sfa, b, sfb)
    exact = gemm.brute_force_exact(a, sfa, b, sfb)
    # fp64 error bound: each promoted term is rounded once and each of the
    # K/128 additions once, so |D64 - exact| <= 2 (K/128) 2^-53 sum_kb |term|.
    da, db = e4m3.decode(a), e4m3.decode(b)
    mag = np.zeros((m, n))
    for kb in range(k // 128):
        sl = slice(kb * 128, (kb + 1) * 128)
        mag += np.abs(da[:, sl] @ db[:, sl].T) * np.abs(sfa[kb, :m, None].astype(np.float64) * sfb[np.arange(n) // 128, kb][None, :])
    for i in range(m):
        for j in range(n):
            bound = Fraction(2 * (k // 128) * 1.0001 * mag[i, j]) * Fraction(1, 2 ** 53)
            assert abs(Fraction(d[i, j]) - exact[i][j]) <= bound


def test_unit_scales_equal_decoded_matmul():
    rng = np.random.default_rng(5)
    m, n, k = 33, 150, 384
    a = rng.integers(0, 256, (m, k), dtype=np.uint8)
    b = rng.integers(0, 256, (n, k), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38  # no NaN codes
    b[(b & 0x7F) == 0x7F] = 0x38
    sfa = np.ones((k // 128, 36), dtype=np.float32)
    sfb = np.ones(((n + 127) // 128, k // 128), dtype=np.float32)
    d = gemm.gemm_nt_ref(a, sfa, b, sfb)
    ta = torch.from_numpy(e4m3.decode(a))
    tb = torch.from_numpy(e4m3.decode(b))
    ref = torch.matmul(ta, tb.T.contiguous()).numpy()  # exact: < 2^25 in 2^-18 steps
    assert np.array_equal(d, ref)


def test_one_hot_activation_selects_weight_column():
    # Row i of A is 1.0 (code 0x38) at column kk[i] and zero elsewhere, sa = 1:
    # D[i][n] = dec(B[n][kk[i]]) * sb[n/128][kk[i]/128], exact and bf16-exact
    # when sb is a power of two.
    m, n, k = 8, 200, 512
    rng = np.random.default_rng(9)
    kk = rng.integers(0, k, m)
    a = np.zeros((m, k), dtype=np.uint8)
    a[np.arange(m), kk] = 0x38
    sfa = np.ones((k // 128, 8), dtype=np.float32)
    b, _ = quant.quant_128x128(bf16_normal((n, k), 3))
    sfb = (2.0 ** rng.integers(-8, 8, ((n + 127) // 128, k // 128))).astype(np.float32)
    d = gemm.gemm_nt_ref(a, sfa, b, sfb)
    expect = e4m3.decode(b[:, kk]).T * sfb[np.arange(n)[None, :] // 128, (kk // 128)[:, None]]
    assert np.array_equal(d, expect)
    assert np.array_equal(bf16.round_f64(d), d)


def test_sign_flip_and_scale_symmetries():
    a, sfa, b, sfb = _operands(16, 136, 384, seed=17)
    d = gemm.gemm_nt_ref(a, sfa, b, sfb)
    assert np.array_equal(gemm.gemm_nt_ref(a ^ 0x80, sfa, b, sfb), -d)
    two = np.float32(2.0 ** 3)
    assert np.array_equal(gemm.gemm_nt_ref(a, sfa * two, b, sfb / two), d)
    assert np.array_equal(gemm.gemm_nt_ref(a, sfa * two, b, sfb), d * 8.0)


def test_partial_sums_per_k_block_are_exact_in_fp64():
    # The argument behind the oracle: |partial| < 128 * 448^2 < 2^25 and every
    # product is a multiple of 2^-18, so 43 bits suffice.  Check the extreme.
    a = np.full((1, 128), 0x7E, dtype=np.uint8)
    b = np.full((1, 128), 0x7E, dtype=np.uint8)
    one = np.ones((1, 4), dtype=np.float32)
    d = gemm.gemm_nt_ref(a, one, b, np.ones((1, 1), dtype=np.float32))
    assert d[0, 0] == 128 * 448.0 ** 2 < 2.0 ** 25
    a2 = np.full((1, 128), 0x01, dtype=np.uint8)  # 2^-9 each
    d2 = gemm.gemm_nt_ref(a2, one, np.concatenate([b[:, :1], a2[:, 1:]], axis=1), np.ones((1, 1), dtype=np.float32))
    assert d2[0, 0] == 2.0 ** -9 * 448.0 + 127 * 2.0 ** -18


def test_contiguous_equals_per_group_dense():
    groups, n, k = 3, 136, 256
    sizes, pads = [128, 256, 0], [0, 0, 128]
    mi = contiguous_m_indices(sizes, pads, order=[1, 0, 2])
    mi[200] = -1  # a padding row inside a block
    mt = mi.size
    a, sfa = quant.quant_1x128(bf16_normal((mt, k), 7))
    b, sfb = quant.quant_128x128(bf16_normal((groups, n, k), 8))
    d, written = gemm.grouped_contiguous_ref(a, sfa, b, sfb, mi)
    assert np.array_equal(written, (mi >= 0) & (mi < groups))
    assert np.all(np.isnan(d[~written]))
    for g in range(groups):
        rows = np.nonzero(mi == g)[0]
        if rows.size:
            assert np.array_equal(d[rows], gemm.gemm_nt_ref(a[rows], sfa[:, rows], b[g], sfb[g]))


def test_group_indexing_pinned_by_distinct_experts():
    # Every A row is 1.0 at k = 0; expert g's weights are (g+1) at k = 0 with
    # unit scales, so D[r][:] = m_indices[r] + 1 exactly on written rows.
    groups, n, k = 4, 64, 128
    mi = contiguous_m_indices([128, 128, 128, 128], order=[2, 0, 3, 1])
    mi[-5:] = -1
    a = np.zeros((mi.size, k), dtype=np.uint8)
    a[:, 0] = 0x38
    sfa = np.ones((1, mi.size), dtype=np.float32)
    b = np.zeros((groups, n, k), dtype=np.uint8)
    codes = [0x38, 0x40, 0x44, 0x48]  # 1, 2, 3, 4
    for g in range(groups):
        b[g, :, 0] = codes[g]
    sfb = np.ones((groups, 1, 1), dtype=np.float32)
    d, written = gemm.grouped_contiguous_ref(a, sfa, b, sfb, mi)
    assert np.array_equal(d[written], np.repeat((mi[written] + 1.0)[:, None], n, axis=1))


@pytest.mark.parametrize("mm", [[0, 1, 127, 128], [129, 200, 300, 7], [-3, 999, 200, 5]])
def test_masked_equals_dense_on_valid_rows(mm):
    groups, m_max, n, k = 4, 200, 136, 256
    a, sfa = quant.quant_1x128(bf16_normal((groups, m_max, k), 12))
    b, sfb = quant.quant_128x128(bf16_normal((groups, n, k), 13))
    d, written = gemm.grouped_masked_ref(a, sfa, b, sfb, np.array(mm))
    for g in range(groups):
        v = min(max(mm[g], 0), m_max)
        assert np.all(written[g, :v]) and not np.any(written[g, v:])
        assert np.all(np.isnan(d[g, v:]))
        if v:
            assert np.array_equal(d[g, :v], gemm.gemm_nt_ref(a[g, :v], sfa[g][:, :v], b[g], sfb[g]))


def test_masked_group_and_row_indexing_pinned_by_closed_form():
    # Independent of gemm_nt_ref: every value below is written out from the
    # operands' construction.  Slice 0: A[g, r, 0] = 1.0 with activation
    # scale (r % 5 + 1) f_g, f_g = 2^(g % 3); expert g's weights are (g + 1)
    # at k = 0 with unit block scale.  Slice 1: A[g, r, 128] = 1.0 with unit
    # scale; B[g][n, 128] = (n % 4 + 1) with block scale h_g = 0.5 (1 + g % 2).
    # So on a valid row
    #     D[g, r, n] = (g + 1)(r % 5 + 1) f_g + h_g (n % 4 + 1)     exactly,
    # which pins the group of every row, the row within the group, the
    # activation-scale group offset and the per-slice weight scale; rows at
    # or past clamp(masked_m[g], 0, M_max) are not written ("DeepGEMM
    # project introduction", Interfaces, Grouped GEMM (masked layout)).
    m_max, n, k = 200, 136, 256
    mm = np.array([-3, 0, 1, 129, m_max, m_max + 7])
    groups = mm.size
    one, codes = 0x38, [0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C]  # 1, 2, 3, 4, 5, 6
    a = np.zeros((groups, m_max, k), dtype=np.uint8)
    a[:, :, 0] = one
    a[:, :, 128] = one
    sfa = np.ones((groups, k // 128, m_max + 4), dtype=np.float32)  # ld > M_max
    f = 2.0 ** (np.arange(groups) % 3)
    h = 0.5 * (1 + np.arange(groups) % 2)
    sfa[:, 0, :m_max] = (np.arange(m_max) % 5 + 1)[None, :] * f[:, None]
    b = np.zeros((groups, n, k), dtype=np.uint8)
    sfb = np.ones((groups, (n + 127) // 128, k // 128), dtype=np.float32)
    for g in range(groups):
        b[g, :, 0] = codes[g]
        b[g, :, 128] = np.array(codes[:4], dtype=np.uint8)[np.arange(n) % 4]
    sfb[:, :, 1] = h[:, None]
    d, written = gemm.grouped_masked_ref(a, sfa, b, sfb, mm)
    r = np.arange(m_max)[:, None]
    c = np.arange(n)[None, :]
    for g in range(groups):
        valid = int(min(max(int(mm[g]), 0), m_max))
        assert np.array_equal(written[g], np.arange(m_max) < valid)
        expect = (g + 1.0) * (r % 5 + 1) * f[g] + h[g] * (c % 4 + 1)
        assert np.array_equal(d[g, :valid], expect[:valid])
        assert np.all(np.isnan(d[g, valid:]))


def test_quantised_gemm_is_close_to_unquantised_product():
    # Gross sanity only (never a parity rule): the quantised product differs
    # from the bf16 product by a few percent, not by zero and not by O(1).
    m, n, k = 64, 256, 1024
    xa, xb = bf16_normal((m, k), 21), bf16_normal((n, k), 22)
    a, sfa = quant.quant_1x128(xa)
    b, sfb = quant.quant_128x128(xb)
    d = gemm.gemm_nt_ref(a, sfa, b, sfb)
    full = bf16.to_f32(xa).astype(np.float64) @ bf16.to_f32(xb).astype(np.float64).T
    rel = np.linalg.norm(d - full) / np.linalg.norm(full)
    assert 5e-3 < rel < 1e-1


def test_tolerance_rule_accepts_bf16_rounding_and_rejects_a_dropped_slice():
    a, sfa, b, sfb = _operands(128, 256, 1024, seed=31)
    d = gemm.gemm_nt_ref(a, sfa, b, sfb)
    check(bf16.round_f64(d), d, "bf16-rounded oracle")
    check(bf16.round_f64(d.astype(np.float32).astype(np.float64)), d, "fp32 then bf16")
    sfa_drop = sfa.copy()
    sfa_drop[3] = 0  # one K slice missing
    with pytest.raises(AssertionError):
        check(bf16.round_f64(gemm.gemm_nt_ref(a, sfa_drop, b, sfb)), d, "dropped slice")
    sfb_t = sfb.copy()
    sfb_t[1] = sfb[0]  # wrong weight-scale block for columns 128..255
    with pytest.raises(AssertionError):
        check(bf16.round_f64(gemm.gemm_nt_ref(a, sfa, b, sfb_t)), d, "wrong sfb block")
