"""GPU parity of every kernel instance, not just the ones the tile heuristic
picks for the shapes above.

DG_FORCE_CONFIG="variant:division:k_rotate" overrides the heuristic (it is
read on every call); division 0 is data-parallel, 1 divides the tiles' K
iterations into equal runs over the grid (stream-K), 3 cuts every tile's K
range into 3 parts.  Each tile variant runs every division, with the K walk
rotated and not, on shapes that are ragged against every tile size
(M = 150, N = 392) with K = 12 slices; the masked and contiguous layouts run
the same sweep.  Both stream-K divisions also run with grid sizes (the
library's CU count) that cut the tiles' K ranges at many different places,
including grids larger than the number of iterations, grids smaller than
the number of parts and grids that are not a multiple of the XCD count.
Every output element is compared with the oracle under the bf16 tolerance
rule.
"""

import numpy as np
import pytest
import torch

from oracle import gemm, quant
from synth import bf16_normal, contiguous_m_indices
from tests.gpu_util import SENTINEL, bf16_to_f64, dev, host, require_gpu
from tests.tolerance import check

pytestmark = pytest.mark.gpu

NUM_VARIANTS = 12
M, N, K = 150, 392, 1536


@pytest.fixture
def force(monkeypatch):
    def _set(variant, division, rotate):
        monkeypatch.setenv("DG_FORCE_CONFIG", f"{variant}:{division}:{rotate}")
    yield _set
    monkeypatch.delenv("DG_FORCE_CONFIG", raising=False)


@pytest.fixture
def num_cus():
    dg = require_gpu()
    yield dg.dg_set_num_cus
    dg.dg_set_num_cus(0)


def _workspace(dg, m, n, k, groups=1):
    size = dg.dg_get_workspace_size(m, n, k, groups)
    return torch.zeros(size, dtype=torch.uint8, device="cuda") if size else None


def _config(dg, layout, m, n, k, groups):
    return dict(kv.split("=") for kv in dg.dg_describe_config(layout, m, n, k, groups, dg.dg_get_num_cus()).split())


@pytest.fixture(scope="module")
def dense_ops():
    xa = bf16_normal((M, K), 501)
    xb = bf16_normal((N, K), 502)
    a, sfa = quant.quant_1x128(xa)
    b, sfb = quant.quant_128x128(xb)
    return a, sfa, b, sfb, gemm.gemm_nt_ref(a, sfa, b, sfb)


def _run_dense(dg, ops, what, ws=None):
    a, sfa, b, sfb, ref = ops
    d = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt(dev(a), dev(sfa), dev(b), dev(sfb), d, workspace=ws if ws is not None else _workspace(dg, M, N, K))
    check(bf16_to_f64(host(d)), ref, what)


@pytest.mark.parametrize("rotate", [0, 1])
@pytest.mark.parametrize("division", [0, 1, 3])
@pytest.mark.parametrize("variant", range(NUM_VARIANTS))
def test_dense_every_variant(variant, division, rotate, force, dense_ops):
    dg = require_gpu()
    force(variant, division, rotate)
    cfg = _config(dg, 0, M, N, K, 1)
    assert int(cfg["variant"]) == variant
    assert int(cfg["stream_k"]) == (division > 0)
    assert int(cfg["sk_split"]) == (division if division >= 2 else 0)
    assert int(cfg["k_rotate"]) == rotate
    _run_dense(dg, dense_ops, f"variant {variant} division {division} rotate {rotate}")


@pytest.mark.parametrize("cus", [1, 3, 13, 40, 200, 1000])
@pytest.mark.parametrize("division", [1, 3])
@pytest.mark.parametrize("variant", [0, 4, 6])
def test_dense_stream_k_grids(variant, division, cus, force, num_cus, dense_ops):
    dg = require_gpu()
    force(variant, division, 1)
    num_cus(cus)
    cfg = _config(dg, 0, M, N, K, 1)
    per_cu = 2 if variant in (4, 7) else 1  # two 64x64 workgroups share a CU
    assert int(cfg["stream_k"]) == 1 and 1 <= int(cfg["grid"]) <= cus * per_cu
    ws = _workspace(dg, M, N, K)
    _run_dense(dg, dense_ops, f"variant {variant} division {division} grid {cfg['grid']}", ws)
    # A second call on the same workspace: every arrival counter was reset.
    _run_dense(dg, dense_ops, f"variant {variant} division {division} grid {cfg['grid']}, second call", ws)


@pytest.mark.parametrize("division", [0, 1, 3])
@pytest.mark.parametrize("variant", range(NUM_VARIANTS))
def test_masked_every_variant(variant, division, force):
    dg = require_gpu()
    force(variant, division, 1)
    g, m_max = 3, 160
    mm = np.array([150, 0, 77], dtype=np.int32)
    xa = bf16_normal((g, m_max, K), 511)
    xb = bf16_normal((g, N, K), 512)
    a, sfa = quant.quant_1x128(xa)
    b, sfb = quant.quant_128x128(xb)
    d = torch.full((g, m_max, N), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_grouped_masked(dev(a), dev(sfa), dev(b), dev(sfb), d, dev(mm), expected_m=int(mm.mean()),
                         workspace=_workspace(dg, m_max, N, K, g))
    out = host(d)
    ref, written = gemm.grouped_masked_ref(a, sfa, b, sfb, mm)
    assert np.all(out[~written] == SENTINEL), f"variant {variant}: rows past masked_m written"
    check(bf16_to_f64(out[written]), ref[written], f"masked variant {variant} division {division}")


@pytest.mark.parametrize("variant", range(NUM_VARIANTS))
def test_contiguous_every_variant(variant, force):
    dg = require_gpu()
    force(variant, 1, 1)  # stream-K is requested but the contiguous layout runs data-parallel
    g = 3
    mi = contiguous_m_indices([128, 384, 256], [0, 128, 0], [2, 0, 1])
    m_total = mi.size
    assert int(_config(dg, 1, m_total, N, K, g)["stream_k"]) == 0
    xa = bf16_normal((m_total, K), 521)
    xb = bf16_normal((g, N, K), 522)
    a, sfa = quant.quant_1x128(xa)
    b, sfb = quant.quant_128x128(xb)
    d = torch.full((m_total, N), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_grouped_contiguous(dev(a), dev(sfa), dev(b), dev(sfb), d, dev(mi.astype(np.int32)),
                             workspace=_workspace(dg, m_total, N, K, g))
    out = host(d)
    ref, written = gemm.grouped_contiguous_ref(a, sfa, b, sfb, mi)
    assert np.all(out[~written] == SENTINEL), f"variant {variant}: padding rows written"
    check(bf16_to_f64(out[written]), ref[written], f"contiguous variant {variant}")
