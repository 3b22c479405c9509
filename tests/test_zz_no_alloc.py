"""The no-allocation dense GEMM (dg_fp8_gemm_nt_noalloc) against the
workspace form (dg_fp8_gemm_nt) and the oracle: two calls in a row on the
library's own scratch, the second smaller and with another configuration,
each equal bit for bit to the workspace form on the same inputs (same
configuration, fixed summation order) and within the bf16 tolerance of the
oracle; a shape needing more scratch than the library holds is refused."""

import numpy as np
import pytest
import torch

from oracle import gemm, quant
from synth import bf16_normal
from tests.gpu_util import SENTINEL, bf16_to_f64, dev, host, require_gpu
from tests.tolerance import check

pytestmark = pytest.mark.gpu


def _operands(m, n, k, seed):
    a, sfa = quant.quant_1x128(bf16_normal((m, k), seed))
    b, sfb = quant.quant_128x128(bf16_normal((n, k), seed + 1))
    return a, sfa, b, sfb


def test_noalloc_matches_workspace_form_on_two_calls():
    dg = require_gpu()
    # 128x2048x16384: 128x128 tiles in 8 K parts; then 64x512x7168: 64x64
    # tiles in 6 parts (a smaller call with another configuration).
    for i, (m, n, k) in enumerate([(128, 2048, 16384), (64, 512, 7168)]):
        desc = dg.dg_describe_config(dg.LAYOUT_DENSE, m, n, k, 1, dg.dg_get_num_cus())
        assert "stream_k=1" in desc, desc  # the scratch is really used
        a, sfa, b, sfb = _operands(m, n, k, seed=5200 + i)
        da, dsfa, db, dsfb = dev(a), dev(sfa), dev(b), dev(sfb)
        got = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
        dg.dg_fp8_gemm_nt_noalloc(da, dsfa, db, dsfb, got)
        ws = torch.zeros(dg.dg_get_workspace_size(m, n, k, 1), dtype=torch.uint8, device="cuda")
        want = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
        dg.dg_fp8_gemm_nt(da, dsfa, db, dsfb, want, workspace=ws)
        torch.cuda.synchronize()
        g, w = host(got), host(want)
        assert np.array_equal(g, w), f"call {i} ({m}x{n}x{k}): differs from dg_fp8_gemm_nt"
        rows = np.arange(0, m, 5)
        check(bf16_to_f64(g[rows]), gemm.gemm_nt_ref(a[rows], sfa[:, rows], b, sfb), f"noalloc call {i}")


def test_noalloc_refuses_shapes_beyond_its_scratch():
    dg = require_gpu()
    m, n, k = 4096, 2816, 7168  # 256x256 tiles in equal K runs: 128 MiB of partials
    assert dg.dg_get_workspace_size(m, n, k, 1) > 33587200
    a = torch.zeros((m, k), dtype=torch.uint8, device="cuda")
    b = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    sfa = torch.zeros((k // 128, dg.dg_get_sf_leading_dim(m)), dtype=torch.float32, device="cuda")
    sfb = torch.zeros(((n + 127) // 128, k // 128), dtype=torch.float32, device="cuda")
    d = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
    with pytest.raises(dg.DGError, match="scratch"):
        dg.dg_fp8_gemm_nt_noalloc(a, sfa, b, sfb, d)
    torch.cuda.synchronize()
    assert bool((d == SENTINEL).all())  # nothing was enqueued
