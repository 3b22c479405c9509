"""GPU parity at the full benchmark sizes, on sampled outputs.

The whole path runs on the GPU as the benchmark runs it: bf16 inputs ->
dg_quant_1x128 / dg_quant_128x128 -> the GEMM entry point.  The oracle then
recomputes, from the same bf16 inputs, the quantisation of sampled A rows and
sampled 128-row weight blocks (both are independent of the rest of the matrix)
and the GEMM restricted to those rows and blocks; the GPU codes and scales on
the samples must match bit for bit and the GPU output on the sampled rows x
block columns must meet the bf16 tolerance rule.  For the masked layout every
row at or past masked_m is checked against a sentinel on the device.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import gemm, quant
from tests.gpu_util import SENTINEL, bf16_to_f64, dev, host, require_gpu
from tests.tolerance import check

pytestmark = pytest.mark.gpu

# The five benchmark workloads and the remaining rows of the pages' tables.
WORKLOADS = synth.workloads() + synth.pages_workloads()


def _sample_rows(rows, count, rng):
    pick = set([0, rows - 1]) | set(rng.integers(0, rows, count).tolist())
    return np.array(sorted(pick))


def _sample_nblocks(n, rng):
    nb = (n + 127) // 128
    return np.array(sorted(set([0, nb - 1, int(rng.integers(0, nb))])))


def _block_rows(n, blocks):
    return np.concatenate([np.arange(b * 128, min(n, (b + 1) * 128)) for b in blocks])


def _same_f32(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


def _quant_b(dg, xb, groups):
    n, k = xb.shape[-2], xb.shape[-1]
    wb = dev(xb)
    qb = torch.empty(xb.shape, dtype=torch.uint8, device="cuda")
    sfb = torch.empty(((groups,) if xb.ndim == 3 else ()) + ((n + 127) // 128, k // 128), dtype=torch.float32, device="cuda")
    dg.dg_quant_128x128(wb, qb, sfb)
    del wb
    return qb, sfb


def _check_b_blocks(qb_h, sfb_h, xb, blocks):
    rows = _block_rows(xb.shape[0], blocks)
    rq, rsf = quant.quant_128x128(xb[rows])
    assert np.array_equal(qb_h[rows], rq)
    assert _same_f32(sfb_h[blocks], rsf)
    return rq, rsf


@pytest.mark.parametrize("wl", [w for w in WORKLOADS if w.layout == "dense"], ids=lambda w: w.name)
def test_dense_workload_sampled(wl):
    dg = require_gpu()
    rng = np.random.default_rng(wl.number * 100 + wl.n)
    m, n, k = wl.m, wl.n, wl.k
    xa = synth.bf16_normal((m, k), wl.seed_a)
    xb = synth.bf16_normal((n, k), wl.seed_b)
    a = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((k // 128, dg.dg_get_sf_leading_dim(m)), dtype=torch.float32, device="cuda")
    dg.dg_quant_1x128(dev(xa), a, sfa)
    qb, sfb = _quant_b(dg, xb, 1)
    ws = dg.dg_get_workspace_size(m, n, k, 1)
    d = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt(a, sfa, qb, sfb, d, workspace=torch.zeros(ws, dtype=torch.uint8, device="cuda") if ws else None)
    torch.cuda.synchronize()

    rows = _sample_rows(m, 12, rng)
    blocks = _sample_nblocks(n, rng)
    cols = _block_rows(n, blocks)
    ra, rsfa = quant.quant_1x128(xa[rows])
    assert np.array_equal(host(a)[rows], ra)
    assert _same_f32(host(sfa)[:, rows], rsfa[:, :rows.size])
    rb, rsfb = _check_b_blocks(host(qb), host(sfb), xb, blocks)
    ref = gemm.gemm_nt_ref(ra, rsfa, rb, rsfb)
    out = host(d)[np.ix_(rows, cols)]
    check(bf16_to_f64(out), ref, wl.name)
    assert not np.any(host(d) == SENTINEL)


@pytest.mark.parametrize("wl", [w for w in WORKLOADS if w.layout == "contiguous"], ids=lambda w: w.name)
def test_contiguous_workload_sampled(wl):
    dg = require_gpu()
    rng = np.random.default_rng(44 + wl.n + wl.groups)
    g, mg, n, k = wl.groups, wl.m, wl.n, wl.k
    m_total = g * mg
    mi = synth.contiguous_m_indices([mg] * g)
    xa = synth.bf16_normal((m_total, k), wl.seed_a)
    xb = synth.bf16_normal((g, n, k), wl.seed_b)
    a = torch.empty((m_total, k), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((k // 128, m_total), dtype=torch.float32, device="cuda")
    dg.dg_quant_1x128(dev(xa), a, sfa)
    qb, sfb = _quant_b(dg, xb, g)
    ws = dg.dg_get_workspace_size(m_total, n, k, g)
    d = torch.full((m_total, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_grouped_contiguous(a, sfa, qb, sfb, d, dev(mi), workspace=torch.zeros(ws, dtype=torch.uint8, device="cuda") if ws else None)
    torch.cuda.synchronize()
    assert not bool((d == SENTINEL).any())

    rows = _sample_rows(m_total, 16, rng)
    a_h, sfa_h = host(a), host(sfa)
    ra, rsfa = quant.quant_1x128(xa[rows])
    assert np.array_equal(a_h[rows], ra)
    assert _same_f32(sfa_h[:, rows], rsfa[:, :rows.size])
    qb_h, sfb_h = host(qb), host(sfb)
    blocks = _sample_nblocks(n, rng)
    cols = _block_rows(n, blocks)
    d_h = host(d)
    for grp in range(g):
        rg = rows[mi[rows] == grp]
        if rg.size == 0:
            continue
        rb, rsfb = _check_b_blocks(qb_h[grp], sfb_h[grp], xb[grp], blocks)
        ra_g, rsfa_g = quant.quant_1x128(xa[rg])
        ref = gemm.gemm_nt_ref(ra_g, rsfa_g, rb, rsfb)
        check(bf16_to_f64(d_h[np.ix_(rg, cols)]), ref, f"{wl.name} group {grp}")


@pytest.mark.parametrize("wl", [w for w in WORKLOADS if w.layout == "masked"], ids=lambda w: w.name)
def test_masked_workload_sampled(wl):
    dg = require_gpu()
    rng = np.random.default_rng(55 + wl.n + wl.groups)
    g, m_max, n, k = wl.groups, wl.m, wl.n, wl.k
    mm = synth.workload_masked_m(wl)
    xa = synth.bf16_normal((g, m_max, k), wl.seed_a)
    xb = synth.bf16_normal((g, n, k), wl.seed_b)
    a = torch.empty((g, m_max, k), dtype=torch.uint8, device="cuda")
    ld = dg.dg_get_sf_leading_dim(m_max)
    sfa = torch.empty((g, k // 128, ld), dtype=torch.float32, device="cuda")
    dg.dg_quant_1x128(dev(xa), a, sfa)
    qb, sfb = _quant_b(dg, xb, g)
    ws = dg.dg_get_workspace_size(m_max, n, k, g)
    d = torch.full((g, m_max, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_grouped_masked(a, sfa, qb, sfb, d, dev(mm), expected_m=int(mm.mean()),
                         workspace=torch.zeros(ws, dtype=torch.uint8, device="cuda") if ws else None)
    torch.cuda.synchronize()

    d_h = host(d)
    a_h, sfa_h, qb_h, sfb_h = host(a), host(sfa), host(qb), host(sfb)
    blocks = _sample_nblocks(n, rng)
    cols = _block_rows(n, blocks)
    for grp in range(g):
        v = int(mm[grp])
        assert np.all(d_h[grp, v:] == SENTINEL), f"group {grp}: rows past masked_m were written"
        assert not np.any(d_h[grp, :v] == SENTINEL)
        rows = _sample_rows(v, 8, rng)
        ra, rsfa = quant.quant_1x128(xa[grp][rows])
        assert np.array_equal(a_h[grp][rows], ra)
        assert _same_f32(sfa_h[grp][:, rows], rsfa[:, :rows.size])
        rb, rsfb = _check_b_blocks(qb_h[grp], sfb_h[grp], xb[grp], blocks)
        ref = gemm.gemm_nt_ref(ra, rsfa, rb, rsfb)
        check(bf16_to_f64(d_h[grp][np.ix_(rows, cols)]), ref, f"{wl.name} group {grp}")
