"""Pins of the K-grouped oracle (oracle/kgrouped.py) against things other than
itself: exact rational brute force, the dense oracle of gemm.py on block-
constant scales, the whole-K sum, the transpose identity and a one-hot closed
form."""

import numpy as np
import pytest

from oracle import e4m3, gemm, kgrouped


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return c


def _scales(rng, kb, rows, ld=None):
    ld = ld or rows
    s = np.zeros((kb, ld), dtype=np.float32)
    s[:, :rows] = rng.uniform(0.25, 4.0, size=(kb, rows)).astype(np.float32) * np.float32(2.0 ** -8)
    return s


def test_brute_force_tiny_with_empty_group():
    rng = np.random.default_rng(5)
    m, n, k = 2, 3, 384
    offs = [0, 128, 128, 384]  # the middle group is empty
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    sfa, sfb = _scales(rng, k // 128, m, 4), _scales(rng, k // 128, n, 4)
    ref = kgrouped.k_grouped_ref(a, sfa, b, sfb, offs)
    exact = kgrouped.k_grouped_brute(a, sfa, b, sfb, offs)
    assert ref.shape == (3, m, n)
    assert np.all(ref[1] == 0.0)
    for g in range(3):
        for i in range(m):
            for j in range(n):
                e = float(exact[g][i][j])
                assert abs(ref[g, i, j] - e) <= 1e-13 * max(1.0, abs(e)), (g, i, j)


def test_groups_equal_dense_oracle_on_block_constant_scales():
    """With B scales constant over each 128-row block, group g is the dense
    NT GEMM of gemm.py over the group's K range."""
    rng = np.random.default_rng(6)
    m, n, k = 5, 200, 1024
    offs = [0, 256, 640, 640, 1024]
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    sfa = _scales(rng, k // 128, m, 8)
    block = _scales(rng, k // 128, (n + 127) // 128)  # [K/128][N/128]
    sfb_rows = np.repeat(block, 128, axis=1)[:, :n]   # [K/128][N], constant per block
    ref = kgrouped.k_grouped_ref(a, sfa, b, sfb_rows, offs)
    for g in range(len(offs) - 1):
        k0, k1 = offs[g], offs[g + 1]
        if k0 == k1:
            assert np.all(ref[g] == 0.0)
            continue
        dense = gemm.gemm_nt_ref(a[:, k0:k1], sfa[k0 // 128:k1 // 128], b[:, k0:k1], block[k0 // 128:k1 // 128].T.copy())
        assert np.allclose(ref[g], dense, rtol=1e-12, atol=1e-12)


def test_groups_sum_to_whole_k():
    rng = np.random.default_rng(7)
    m, n, k = 4, 6, 1280
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    sfa, sfb = _scales(rng, k // 128, m), _scales(rng, k // 128, n)
    parts = kgrouped.k_grouped_ref(a, sfa, b, sfb, [0, 384, 512, 1280])
    whole = kgrouped.k_grouped_ref(a, sfa, b, sfb, [0, 1280])
    assert np.allclose(parts.sum(axis=0), whole[0], rtol=1e-12, atol=1e-12)


def test_transpose_identity():
    rng = np.random.default_rng(8)
    m, n, k = 3, 7, 512
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    sfa, sfb = _scales(rng, k // 128, m), _scales(rng, k // 128, n)
    offs = [0, 128, 512]
    d = kgrouped.k_grouped_ref(a, sfa, b, sfb, offs)
    dt = kgrouped.k_grouped_ref(b, sfb, a, sfa, offs)
    assert np.array_equal(d, np.transpose(dt, (0, 2, 1)))


def test_one_hot_closed_form():
    m, n, k = 2, 2, 512
    a = np.zeros((m, k), dtype=np.uint8)
    b = np.zeros((n, k), dtype=np.uint8)
    a[1, 300] = 0x40   # 2.0
    b[0, 300] = 0xC8   # -4.0
    sfa = np.full((k // 128, m), 0.5, dtype=np.float32)
    sfb = np.full((k // 128, n), 0.25, dtype=np.float32)
    sfa[2, 1] = 3.0    # slice 2 holds k = 300
    sfb[2, 0] = 0.125
    assert e4m3.decode(np.array([0x40, 0xC8], dtype=np.uint8)).tolist() == [2.0, -4.0]
    d = kgrouped.k_grouped_ref(a, sfa, b, sfb, [0, 256, 512])
    want = np.zeros((2, m, n))
    want[1, 1, 0] = 2.0 * -4.0 * 3.0 * 0.125  # group 1 holds k in [256, 512)
    assert np.array_equal(d, want)


@pytest.mark.parametrize("offs", [[0, 128, 384], [128, 512], [0, 256, 200, 512], [0, 100, 512]])
def test_bad_offsets_rejected(offs):
    a = np.zeros((1, 512), dtype=np.uint8)
    s = np.ones((4, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        kgrouped.k_grouped_ref(a, s, a, s, offs)
