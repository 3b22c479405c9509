"""Pins of oracle/majors.py against things other than itself: an exact
rational brute force that indexes the stored arrays directly (no transposed
views), one-hot closed forms in every layout on non-square shapes (a swapped
operand or transposition moves or loses the single non-zero), the NT layout
reducing to gemm.py, and the column quantiser against the row quantiser of
the transposed matrix plus its own invariants."""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import e4m3, gemm, majors, quant, ue8m0

LAYOUTS = ["nt", "nn", "tn", "tt"]


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return c


def _stored(layout, a_log, b_log):
    """Stored arrays for logical A [M][K], B [N][K], built element by element."""
    m, k = a_log.shape
    n = b_log.shape[0]
    a = np.zeros((m, k) if layout[0] == "n" else (k, m), dtype=np.uint8)
    b = np.zeros((n, k) if layout[1] == "t" else (k, n), dtype=np.uint8)
    for i in range(m):
        for kk in range(k):
            if layout[0] == "n":
                a[i, kk] = a_log[i, kk]
            else:
                a[kk, i] = a_log[i, kk]
    for j in range(n):
        for kk in range(k):
            if layout[1] == "t":
                b[j, kk] = b_log[j, kk]
            else:
                b[kk, j] = b_log[j, kk]
    return a, b


def _brute(layout, a, sfa, b, sfb, m, n, k):
    """Exact D from the stored arrays, reading A(i, kk) and B(j, kk) by index."""
    dec = [Fraction(e4m3.decode_one(c)) if (c & 0x7F) != 0x7F else None for c in range(256)]
    a_at = (lambda i, kk: a[i, kk]) if layout[0] == "n" else (lambda i, kk: a[kk, i])
    b_at = (lambda j, kk: b[j, kk]) if layout[1] == "t" else (lambda j, kk: b[kk, j])
    out = np.zeros((m, n), dtype=object)
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for kb in range(k // 128):
                part = sum((dec[int(a_at(i, kk))] * dec[int(b_at(j, kk))] for kk in range(kb * 128, kb * 128 + 128)),
                           Fraction(0))
                tot += part * Fraction(float(sfa[kb][i])) * Fraction(float(sfb[j // 128][kb]))
            out[i, j] = tot
    return out


@pytest.mark.parametrize("layout", LAYOUTS)
def test_brute_force_tiny(layout):
    rng = np.random.default_rng(40 + LAYOUTS.index(layout))
    m, n, k = 3, 5, 256
    a_log, b_log = _codes(rng, (m, k)), _codes(rng, (n, k))
    a, b = _stored(layout, a_log, b_log)
    sfa = np.zeros((k // 128, 4), dtype=np.float32)
    sfa[:, :m] = rng.uniform(0.25, 4, (k // 128, m)) * 2.0 ** -8
    sfb = (rng.uniform(0.25, 4, (1, k // 128)) * 2.0 ** -8).astype(np.float32)
    ref = majors.gemm_layout_ref(layout, a, sfa, b, sfb)
    exact = _brute(layout, a, sfa, b, sfb, m, n, k)
    for i in range(m):
        for j in range(n):
            e = float(exact[i, j])
            assert abs(ref[i, j] - e) <= 1e-13 * max(1.0, abs(e)), (layout, i, j)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_one_hot_closed_form(layout):
    """One non-zero code in A at logical (5, 300), one in B at logical (70, 300):
    D is zero except D[5][70] = 2 * -4 * sa * sb, in every layout."""
    m, n, k = 48, 80, 384
    a_log = np.zeros((m, k), dtype=np.uint8)
    b_log = np.zeros((n, k), dtype=np.uint8)
    a_log[5, 300] = 0x40  # 2.0
    b_log[70, 300] = 0xC8  # -4.0
    a, b = _stored(layout, a_log, b_log)
    sfa = np.full((k // 128, m), 0.5, dtype=np.float32)
    sfb = np.full((1, k // 128), 0.25, dtype=np.float32)
    sfa[2, 5] = 3.0
    sfb[0, 2] = 0.125
    d = majors.gemm_layout_ref(layout, a, sfa, b, sfb)
    want = np.zeros((m, n))
    want[5, 70] = 2.0 * -4.0 * 3.0 * 0.125
    assert np.array_equal(d, want)


def test_nt_is_the_plain_gemm():
    rng = np.random.default_rng(44)
    a, b = _codes(rng, (4, 256)), _codes(rng, (130, 256))
    sfa = (rng.uniform(0.5, 2, (2, 4)) * 2.0 ** -8).astype(np.float32)
    sfb = (rng.uniform(0.5, 2, (2, 2)) * 2.0 ** -8).astype(np.float32)
    assert np.array_equal(majors.gemm_layout_ref("nt", a, sfa, b, sfb), gemm.gemm_nt_ref(a, sfa, b, sfb))


def test_bad_layout_rejected():
    with pytest.raises(ValueError):
        majors.logical_operands("xn", np.zeros((1, 128)), np.zeros((1, 128)))


@pytest.mark.parametrize("k,m,ld", [(256, 40, None), (128, 8, 16), (384, 136, 140)])
def test_column_quantiser_is_row_quantiser_of_transpose(k, m, ld):
    x = synth.bf16_normal((k, m), 45 + m)
    x[128:256 if k > 128 else 128, 3] = 0       # an all-zero column tile (when K allows)
    x[0:128, 1] = 0x8000                          # a tile of -0 only
    q, sf = majors.quant_1x128_mn(x, ld)
    qt, sft = quant.quant_1x128(np.ascontiguousarray(x.T), ld)
    assert np.array_equal(q, qt.T)
    assert np.array_equal(sf.view(np.uint32), sft.view(np.uint32))
    assert np.all(q[0:128, 1] == 0x80)


def test_column_quantiser_invariants():
    """Each non-zero column tile holds a +-448 code (0x7E / 0xFE) at its amax
    element, and dequantised values are within half an e4m3 step."""
    k, m = 256, 24
    x = synth.bf16_normal((k, m), 46)
    q, sf = majors.quant_1x128_mn(x)
    xf = np.asarray(x, dtype=np.uint32).astype(np.uint32) << 16
    xv = xf.view(np.float32).astype(np.float64)
    deq = e4m3.decode(q)
    for kb in range(k // 128):
        seg = xv[kb * 128:(kb + 1) * 128]
        for c in range(m):
            r = int(np.argmax(np.abs(seg[:, c])))
            assert q[kb * 128 + r, c] & 0x7F == 0x7E
            err = np.abs(deq[kb * 128:(kb + 1) * 128, c] * sf[kb, c] - seg[:, c])
            assert np.all(err <= 2.0 ** -4 * np.abs(seg[:, c]) + 2.0 ** -10 * sf[kb, c])


@pytest.mark.parametrize("k,m,ld", [(256, 40, None), (128, 8, 16)])
def test_column_ue8m0_quantiser_is_row_quantiser_of_transpose(k, m, ld):
    x = synth.bf16_normal((k, m), 47 + m)
    x[0:128, 3] = 0          # all-zero column tile: E = 0
    x[0:128, 5] = 0x43E0     # 448 everywhere: E = 127
    q, sf = majors.quant_1x128_mn_ue8m0(x, ld)
    qt, sft = ue8m0.quant_1x128_ue8m0(np.ascontiguousarray(x.T), ld)
    assert np.array_equal(q, qt.T)
    assert np.array_equal(sf, sft)
    assert sf[0, 3] == 0 and sf[0, 5] == 127
