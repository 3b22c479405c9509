"""GPU parity of every kernel instance, not just the ones the tile heuristic
picks for the shapes above.

DG_FORCE_CONFIG="variant:split_k:k_rotate" overrides the heuristic (it is
read on every call).  Each tile variant runs unsplit and with K split three
ways, with the K walk rotated and not, on shapes that are ragged against
every tile size (M = 150, N = 392) and whose K (12 slices) splits unevenly
with rotation; the masked and contiguous layouts run the same sweep.  Every
output element is compared with the oracle under the bf16 tolerance rule.
"""


import numpy as np
import pytest
import torch

from oracle import gemm, quant
from synth import bf16_normal, contiguous_m_indices
from tests.gpu_util import SENTINEL, bf16_to_f64, dev, host, require_gpu
from tests.tolerance import check

pytestmark = pytest.mark.gpu

NUM_VARIANTS = 11
M, N, K = 150, 392, 1536


@pytest.fixture
def force(monkeypatch):
    def _set(variant, split, rotate):
        monkeypatch.setenv("DG_FORCE_CONFIG", f"{variant}:{split}:{rotate}")
    yield _set
    monkeypatch.delenv("DG_FORCE_CONFIG", raising=False)


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


@pytest.mark.parametrize("rotate", [0, 1])
@pytest.mark.parametrize("split", [1, 3])
@pytest.mark.parametrize("variant", range(NUM_VARIANTS))
def test_dense_every_variant(variant, split, rotate, force, dense_ops):
    dg = require_gpu()
    force(variant, split, rotate)
    cfg = _config(dg, 0, M, N, K, 1)
    assert int(cfg["variant"]) == variant
    assert int(cfg["k_rotate"]) == rotate
    a, sfa, b, sfb, ref = dense_ops
    d = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt(dev(a), dev(sfa), dev(b), dev(sfb), d, workspace=_workspace(dg, M, N, K))
    check(bf16_to_f64(host(d)), ref, f"variant {variant} split {cfg['split_k']} rotate {rotate}")


@pytest.mark.parametrize("split", [1, 3])
@pytest.mark.parametrize("variant", range(NUM_VARIANTS))
def test_masked_every_variant(variant, split, force):
    dg = require_gpu()
    force(variant, split, 1)
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
    check(bf16_to_f64(out[written]), ref[written], f"masked variant {variant}")


@pytest.mark.parametrize("variant", range(NUM_VARIANTS))
def test_contiguous_every_variant(variant, force):
    dg = require_gpu()
    force(variant, 1, 1)
    g = 3
    mi = contiguous_m_indices([128, 384, 256], [0, 128, 0], [2, 0, 1])
    m_total = mi.size
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
