"""GPU parity of the power-of-two (UE8M0) scale path.

Quantisers: the e4m3 codes and the exponent bytes (padding included) must
equal the oracle's bit for bit.  GEMMs: the GPU output is compared with the
oracle's reference GEMM, fed the oracle's exponents turned into the fp32
powers of two they stand for, under the bf16 tolerance rule: on ragged small
shapes for every UE8M0 tile instance and work division, and on sampled
outputs of the benchmark workloads at full size.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import gemm, ue8m0
from synth import bf16_normal, contiguous_m_indices
from tests.gpu_util import (SENTINEL, bf16_to_f64, dev, gpu_quant_1x128_ue8m0, gpu_quant_128x128_ue8m0,
                            host, require_gpu)
from tests.tolerance import check

pytestmark = pytest.mark.gpu

UE8M0_VARIANTS = [0, 1, 4, 5, 6]
M, N, K = 150, 392, 1536


def _ref_ops(xa, xb):
    """Oracle quantisation of bf16 A [M][K] and B [N][K]: (a, sfa, b, sfb) with
    the exponents as fp32 scales in the layout gemm.py consumes."""
    a, ea = ue8m0.quant_1x128_ue8m0(xa)
    b, eb = ue8m0.quant_128x128_ue8m0(xb)
    return a, ea, b, eb


def _ws(dg, m, n, k, groups=1):
    size = dg.dg_get_workspace_size(m, n, k, groups)
    return torch.zeros(size, dtype=torch.uint8, device="cuda") if size else None


# ------------------------------------------------------------ quantisers --

@pytest.mark.parametrize("rows,cols", [(1, 128), (5, 256), (33, 384), (64, 7168), (130, 1536), (1000, 512)])
def test_quant_1x128_ue8m0_bit_exact(rows, cols):
    dg = require_gpu()
    x = bf16_normal((rows, cols), seed=600 + rows)
    q, sf = gpu_quant_1x128_ue8m0(dg, x)
    rq, rsf = ue8m0.quant_1x128_ue8m0(x)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(sf), rsf)


# Heights around the quantiser's rows-per-trip thresholds, ragged last trips,
# and group boundaries inside a four-row trip.
@pytest.mark.parametrize("shape", [(2051, 384), (16395, 256), (3, 5467, 128)])
def test_quant_1x128_ue8m0_tall_bit_exact(shape):
    dg = require_gpu()
    x = bf16_normal(shape, seed=610 + shape[-2])
    ld = 5480 if len(shape) == 3 else None
    q, sf = gpu_quant_1x128_ue8m0(dg, x, ld=ld)
    rq, rsf = ue8m0.quant_1x128_ue8m0(x, ld_sf=ld) if ld else ue8m0.quant_1x128_ue8m0(x)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(sf), rsf)


def test_quant_1x128_ue8m0_grouped_and_wide_ld():
    dg = require_gpu()
    x = bf16_normal((3, 37, 256), seed=78)
    q, sf = gpu_quant_1x128_ue8m0(dg, x, ld=48)
    rq, rsf = ue8m0.quant_1x128_ue8m0(x, ld_sf=48)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(sf), rsf)


def _special_tiles():
    x = bf16_normal((8, 512), seed=89)
    x[0, 0:128] = 0x0000                      # all +0: E = 0
    x[1, 128:256] = 0x8000                    # all -0
    x[2, 256:384] = 0
    x[2, 256] = 0x0380                        # amax 2^-120: E clamps to 0
    x[3, 0:128] = 0
    x[3, 5] = 0x0001                          # smallest bf16 subnormal
    x[4, 384:512] = np.arange(128, dtype=np.uint16) | 0x0001
    x[5, 0:128] = 0x43E0                      # 448 everywhere: E = 127 exactly
    x[6, 0:128] = 0x43E1                      # just above 448: E = 128
    x[7, 128:256] = 0x7F7F                    # bf16 max: E = 247
    x[7, 256:384] = 0xFF7F                    # -bf16 max
    return x


def test_quant_1x128_ue8m0_special_tiles():
    dg = require_gpu()
    x = _special_tiles()
    q, sf = gpu_quant_1x128_ue8m0(dg, x)
    rq, rsf = ue8m0.quant_1x128_ue8m0(x)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(sf), rsf)


@pytest.mark.parametrize("rows,cols", [(128, 128), (200, 384), (7168, 512), (1, 256), (513, 1024)])
def test_quant_128x128_ue8m0_bit_exact(rows, cols):
    dg = require_gpu()
    w = bf16_normal((rows, cols), seed=700 + rows)
    q, sf = gpu_quant_128x128_ue8m0(dg, w)
    rq, rsf = ue8m0.quant_128x128_ue8m0(w)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(sf), rsf)


def test_quant_128x128_ue8m0_grouped_special():
    dg = require_gpu()
    w = bf16_normal((3, 300, 384), seed=79)
    w[0, 0:128, 0:128] = 0                    # zero block
    w[1, 256:300, 128:256] = 0x43E0           # ragged last block at 448
    w[2, 5, 256] = 0x7F7F                     # one huge value in a block
    q, sf = gpu_quant_128x128_ue8m0(dg, w)
    rq, rsf = ue8m0.quant_128x128_ue8m0(w)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(sf), rsf)


# ------------------------------------------------------------------ GEMMs --

@pytest.fixture(scope="module")
def dense_ops():
    xa = bf16_normal((M, K), 601)
    xb = bf16_normal((N, K), 602)
    a, ea, b, eb = _ref_ops(xa, xb)
    return a, ea, b, eb, gemm.gemm_nt_ref(a, ue8m0.sfa_as_fp32(ea), b, ue8m0.sfb_as_fp32(eb, N))


@pytest.fixture
def force(monkeypatch):
    def _set(variant, division, rotate):
        monkeypatch.setenv("DG_FORCE_CONFIG", f"{variant}:{division}:{rotate}")
    yield _set
    monkeypatch.delenv("DG_FORCE_CONFIG", raising=False)


def _run_dense(dg, ops, what):
    a, ea, b, eb, ref = ops
    d = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt_ue8m0(dev(a), dev(ea), dev(b), dev(eb), d, workspace=_ws(dg, M, N, K))
    check(bf16_to_f64(host(d)), ref, what)


def test_dense_default_config(dense_ops):
    dg = require_gpu()
    _run_dense(dg, dense_ops, "ue8m0 dense default")


@pytest.mark.parametrize("rotate", [0, 1])
@pytest.mark.parametrize("division", [0, 1, 3])
@pytest.mark.parametrize("variant", UE8M0_VARIANTS)
def test_dense_every_variant(variant, division, rotate, force, dense_ops):
    dg = require_gpu()
    force(variant, division, rotate)
    _run_dense(dg, dense_ops, f"ue8m0 variant {variant} division {division} rotate {rotate}")


def test_unbuilt_variant_is_rejected(force, dense_ops):
    dg = require_gpu()
    force(2, 0, 0)
    a, ea, b, eb, _ = dense_ops
    d = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda")
    with pytest.raises(dg.DGError) as err:
        dg.dg_fp8_gemm_nt_ue8m0(dev(a), dev(ea), dev(b), dev(eb), d, workspace=_ws(dg, M, N, K))
    assert err.value.status == -2
    torch.cuda.synchronize()
    assert bool((d == SENTINEL).all())


def test_dense_extreme_exponents():
    """Scales far from 1: exponents near both ends of the range the quantisers
    produce, so the block-scaled product reaches tiny and huge magnitudes."""
    dg = require_gpu()
    m, n, k = 64, 256, 512
    xa = bf16_normal((m, k), 611, scale=2.0 ** 60)
    xb = bf16_normal((n, k), 612, scale=2.0 ** -70)
    a, ea, b, eb = _ref_ops(xa, xb)
    ref = gemm.gemm_nt_ref(a, ue8m0.sfa_as_fp32(ea), b, ue8m0.sfb_as_fp32(eb, n))
    d = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt_ue8m0(dev(a), dev(ea), dev(b), dev(eb), d, workspace=_ws(dg, m, n, k))
    check(bf16_to_f64(host(d)), ref, "ue8m0 extreme exponents")


@pytest.mark.parametrize("division", [0, 1, 3])
@pytest.mark.parametrize("variant", UE8M0_VARIANTS)
def test_masked_every_variant(variant, division, force):
    dg = require_gpu()
    force(variant, division, 1)
    g, m_max = 3, 160
    mm = np.array([150, 0, 77], dtype=np.int32)
    xa = bf16_normal((g, m_max, K), 621)
    xb = bf16_normal((g, N, K), 622)
    a, ea = ue8m0.quant_1x128_ue8m0(xa)
    b, eb = ue8m0.quant_128x128_ue8m0(xb)
    d = torch.full((g, m_max, N), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_grouped_masked_ue8m0(dev(a), dev(ea), dev(b), dev(eb), d, dev(mm), expected_m=int(mm.mean()),
                               workspace=_ws(dg, m_max, N, K, g))
    out = host(d)
    ref, written = gemm.grouped_masked_ref(a, ue8m0.sfa_as_fp32(ea), b, ue8m0.sfb_as_fp32(eb, N), mm)
    assert np.all(out[~written] == SENTINEL), f"variant {variant}: rows past masked_m written"
    check(bf16_to_f64(out[written]), ref[written], f"ue8m0 masked variant {variant} division {division}")


@pytest.mark.parametrize("variant", UE8M0_VARIANTS)
def test_contiguous_every_variant(variant, force):
    dg = require_gpu()
    force(variant, 0, 1)
    g = 3
    mi = contiguous_m_indices([128, 384, 256], [0, 128, 0], [2, 0, 1])
    m_total = mi.size
    xa = bf16_normal((m_total, K), 631)
    xb = bf16_normal((g, N, K), 632)
    a, ea = ue8m0.quant_1x128_ue8m0(xa)
    b, eb = ue8m0.quant_128x128_ue8m0(xb)
    d = torch.full((m_total, N), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_grouped_contiguous_ue8m0(dev(a), dev(ea), dev(b), dev(eb), d, dev(mi.astype(np.int32)),
                                   workspace=_ws(dg, m_total, N, K, g))
    out = host(d)
    ref, written = gemm.grouped_contiguous_ref(a, ue8m0.sfa_as_fp32(ea), b, ue8m0.sfb_as_fp32(eb, N), mi)
    assert np.all(out[~written] == SENTINEL), f"variant {variant}: padding rows written"
    check(bf16_to_f64(out[written]), ref[written], f"ue8m0 contiguous variant {variant}")


# ----------------------------------------------- full sizes, sampled outputs --

def _sample_rows(rows, count, rng):
    return np.array(sorted(set([0, rows - 1]) | set(rng.integers(0, rows, count).tolist())))


def _sample_nblocks(n, rng):
    nb = (n + 127) // 128
    return np.array(sorted(set([0, nb - 1, int(rng.integers(0, nb))])))


def _block_rows(n, blocks):
    return np.concatenate([np.arange(b * 128, min(n, (b + 1) * 128)) for b in blocks])


def _gpu_quant_a(dg, xa, ld):
    a = torch.empty(xa.shape, dtype=torch.uint8, device="cuda")
    shape = (xa.shape[-1] // 128, ld) if xa.ndim == 2 else (xa.shape[0], xa.shape[-1] // 128, ld)
    ea = torch.empty(shape, dtype=torch.uint8, device="cuda")
    dg.dg_quant_1x128_ue8m0(dev(xa), a, ea)
    return a, ea


def _gpu_quant_b(dg, xb):
    n, k = xb.shape[-2], xb.shape[-1]
    b = torch.empty(xb.shape, dtype=torch.uint8, device="cuda")
    shape = (k // 128, dg.dg_get_ue8m0_sfb_leading_dim(n))
    eb = torch.empty(((xb.shape[0],) if xb.ndim == 3 else ()) + shape, dtype=torch.uint8, device="cuda")
    dg.dg_quant_128x128_ue8m0(dev(xb), b, eb)
    return b, eb


def _check_samples(a_h, ea_h, b_h, eb_h, xa, xb, rows, blocks):
    """Bit-exact quantisation of the sampled rows and blocks; returns the
    oracle's operands restricted to them."""
    ra, rea = ue8m0.quant_1x128_ue8m0(xa[rows])
    assert np.array_equal(a_h[rows], ra)
    assert np.array_equal(ea_h[:, rows], rea[:, :rows.size])
    brows = _block_rows(xb.shape[0], blocks)
    rb, reb = ue8m0.quant_128x128_ue8m0(xb[brows])
    assert np.array_equal(b_h[brows], rb)
    assert np.array_equal(eb_h[:, blocks], reb[:, :blocks.size])
    return ra, ue8m0.sfa_as_fp32(rea), rb, ue8m0.sfb_as_fp32(reb, brows.size)


@pytest.mark.parametrize("wl", synth.workloads(), ids=lambda w: w.name)
def test_workload_sampled(wl):
    dg = require_gpu()
    rng = np.random.default_rng(900 + wl.number * 10 + wl.n % 97)
    g, m, n, k = wl.groups, wl.m, wl.n, wl.k
    if wl.layout == "dense":
        xa = synth.bf16_normal((m, k), wl.seed_a)
        xb = synth.bf16_normal((n, k), wl.seed_b)
        a, ea = _gpu_quant_a(dg, xa, dg.dg_get_sf_leading_dim(m))
        b, eb = _gpu_quant_b(dg, xb)
        d = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
        dg.dg_fp8_gemm_nt_ue8m0(a, ea, b, eb, d, workspace=_ws(dg, m, n, k))
        torch.cuda.synchronize()
        rows, blocks = _sample_rows(m, 12, rng), _sample_nblocks(n, rng)
        ops = _check_samples(host(a), host(ea), host(b), host(eb), xa, xb, rows, blocks)
        check(bf16_to_f64(host(d)[np.ix_(rows, _block_rows(n, blocks))]), gemm.gemm_nt_ref(*ops), wl.name)
        assert not bool((d == SENTINEL).any())
    elif wl.layout == "contiguous":
        m_total = g * m
        mi = synth.contiguous_m_indices([m] * g)
        xa = synth.bf16_normal((m_total, k), wl.seed_a)
        xb = synth.bf16_normal((g, n, k), wl.seed_b)
        a, ea = _gpu_quant_a(dg, xa, m_total)
        b, eb = _gpu_quant_b(dg, xb)
        d = torch.full((m_total, n), SENTINEL, dtype=torch.int16, device="cuda")
        dg.dg_grouped_contiguous_ue8m0(a, ea, b, eb, d, dev(mi), workspace=_ws(dg, m_total, n, k, g))
        torch.cuda.synchronize()
        assert not bool((d == SENTINEL).any())
        a_h, ea_h, b_h, eb_h, d_h = host(a), host(ea), host(b), host(eb), host(d)
        rows, blocks = _sample_rows(m_total, 16, rng), _sample_nblocks(n, rng)
        for grp in range(g):
            rg = rows[mi[rows] == grp]
            if rg.size:
                ops = _check_samples(a_h, ea_h, b_h[grp], eb_h[grp], xa, xb[grp], rg, blocks)
                check(bf16_to_f64(d_h[np.ix_(rg, _block_rows(n, blocks))]), gemm.gemm_nt_ref(*ops),
                      f"{wl.name} group {grp}")
    else:
        mm = synth.workload_masked_m(wl)
        xa = synth.bf16_normal((g, m, k), wl.seed_a)
        xb = synth.bf16_normal((g, n, k), wl.seed_b)
        a, ea = _gpu_quant_a(dg, xa, dg.dg_get_sf_leading_dim(m))
        b, eb = _gpu_quant_b(dg, xb)
        d = torch.full((g, m, n), SENTINEL, dtype=torch.int16, device="cuda")
        dg.dg_grouped_masked_ue8m0(a, ea, b, eb, d, dev(mm), expected_m=int(mm.mean()),
                                   workspace=_ws(dg, m, n, k, g))
        torch.cuda.synchronize()
        a_h, ea_h, b_h, eb_h, d_h = host(a), host(ea), host(b), host(eb), host(d)
        blocks = _sample_nblocks(n, rng)
        for grp in range(g):
            v = int(mm[grp])
            assert np.all(d_h[grp, v:] == SENTINEL), f"group {grp}: rows past masked_m were written"
            assert not np.any(d_h[grp, :v] == SENTINEL)
            if v == 0:
                continue
            rows = _sample_rows(v, 8, rng)
            ops = _check_samples(a_h[grp], ea_h[grp], b_h[grp], eb_h[grp], xa[grp], xb[grp], rows, blocks)
            check(bf16_to_f64(d_h[grp][np.ix_(rows, _block_rows(n, blocks))]), gemm.gemm_nt_ref(*ops),
                  f"{wl.name} group {grp}")
