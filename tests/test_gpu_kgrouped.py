"""GPU parity of the K-grouped GEMM (dg_k_grouped_nt) against oracle/kgrouped.py.

Both operands are quantised per 1x128 tile along K (the oracle's activation
quantiser); every group's output is compared with the oracle under the bf16
tolerance rule, empty groups must be exact zeros, and on exact-grid inputs
(every scale 2^-8, the fp32 result exact in any order) the output must equal
the oracle's bf16 rounding bit for bit.  Each K-grouped tile instance runs;
a realistic weight-gradient shape runs at full size on sampled rows and
columns; out-of-contract offsets are clamped without reading out of bounds.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import bf16, kgrouped, quant
from tests.gpu_util import SENTINEL, bf16_to_f64, dev, host, require_gpu
from tests.tolerance import check

pytestmark = pytest.mark.gpu

KG_VARIANTS = [0, 4, 5, 6]


def _operands(xa, xb):
    a, sfa = quant.quant_1x128(xa)
    b, sfb = quant.quant_1x128(xb)
    return a, sfa, b, sfb


def _run(dg, a, sfa, b, sfb, offs, groups):
    m, n = a.shape[0], b.shape[0]
    d = torch.full((groups, m, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_k_grouped_nt(dev(a), dev(sfa), dev(b), dev(sfb), d, dev(np.asarray(offs, dtype=np.int32)))
    return host(d)


@pytest.fixture
def force(monkeypatch):
    def _set(variant):
        monkeypatch.setenv("DG_FORCE_CONFIG", f"{variant}:0:0")
    yield _set
    monkeypatch.delenv("DG_FORCE_CONFIG", raising=False)


M, N, K = 150, 392, 1536
OFFS = [0, 384, 384, 1152, 1536]  # group 1 is empty


@pytest.fixture(scope="module")
def random_ops():
    a, sfa, b, sfb = _operands(synth.bf16_normal((M, K), 901), synth.bf16_normal((N, K), 902))
    return a, sfa, b, sfb, kgrouped.k_grouped_ref(a, sfa, b, sfb, OFFS)


def _check_groups(out, ref, what):
    for g in range(ref.shape[0]):
        if np.all(ref[g] == 0):
            assert np.all(out[g] == 0), f"{what}: empty group {g} not zero"
        else:
            check(bf16_to_f64(out[g]), ref[g], f"{what} group {g}")


def test_default_config(random_ops):
    dg = require_gpu()
    a, sfa, b, sfb, ref = random_ops
    _check_groups(_run(dg, a, sfa, b, sfb, OFFS, 4), ref, "k-grouped default")


@pytest.mark.parametrize("variant", KG_VARIANTS)
def test_every_variant(variant, force, random_ops):
    dg = require_gpu()
    force(variant)
    a, sfa, b, sfb, ref = random_ops
    _check_groups(_run(dg, a, sfa, b, sfb, OFFS, 4), ref, f"k-grouped variant {variant}")


@pytest.mark.parametrize("variant", KG_VARIANTS)
def test_exact_grid_bitwise(variant, force):
    dg = require_gpu()
    force(variant)
    m, n, k = 200, 264, 1024
    offs = [0, 128, 640, 1024]
    a, sfa, b, sfb = _operands(synth.bf16_grid((m, k), 911), synth.bf16_grid((n, k), 912))
    ref = kgrouped.k_grouped_ref(a, sfa, b, sfb, offs)
    assert np.all(ref * 16 == np.round(ref * 16)) and np.abs(ref).max() < 2.0 ** 19
    out = _run(dg, a, sfa, b, sfb, offs, 3)
    assert np.array_equal(out, bf16.bits_from_f64(ref))


def test_unbuilt_variant_is_rejected(force, random_ops):
    dg = require_gpu()
    force(2)
    a, sfa, b, sfb, _ = random_ops
    with pytest.raises(dg.DGError) as err:
        _run(dg, a, sfa, b, sfb, OFFS, 4)
    assert err.value.status == -2


def test_offsets_are_clamped():
    """Out-of-contract offsets (not multiples of 128, beyond K) are clamped to
    [0, K] and rounded down to a slice: [0, 100, 9999] acts as [0, 0, K]."""
    dg = require_gpu()
    m, n, k = 64, 128, 512
    a, sfa, b, sfb = _operands(synth.bf16_normal((m, k), 921), synth.bf16_normal((n, k), 922))
    ref = kgrouped.k_grouped_ref(a, sfa, b, sfb, [0, 0, k])
    _check_groups(_run(dg, a, sfa, b, sfb, [0, 100, 9999], 2), ref, "clamped offsets")


def test_weight_gradient_shape_sampled():
    """8 experts with unequal token counts (K = 8192 in all), M = 7168, N = 2048:
    the oracle recomputes sampled rows and columns of every group."""
    dg = require_gpu()
    rng = np.random.default_rng(931)
    m, n = 7168, 2048
    tokens = [1024, 640, 1536, 0, 1152, 2048, 896, 896]
    offs = np.concatenate([[0], np.cumsum(tokens)]).astype(np.int32)
    k = int(offs[-1])
    xa = synth.bf16_normal((m, k), 932)
    xb = synth.bf16_normal((n, k), 933)
    a = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((k // 128, dg.dg_get_sf_leading_dim(m)), dtype=torch.float32, device="cuda")
    b = torch.empty((n, k), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((k // 128, dg.dg_get_sf_leading_dim(n)), dtype=torch.float32, device="cuda")
    dg.dg_quant_1x128(dev(xa), a, sfa)
    dg.dg_quant_1x128(dev(xb), b, sfb)
    g = len(tokens)
    d = torch.full((g, m, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_k_grouped_nt(a, sfa, b, sfb, d, dev(offs))
    torch.cuda.synchronize()
    rows = np.array(sorted(set([0, m - 1]) | set(rng.integers(0, m, 10).tolist())))
    cols = np.array(sorted(set([0, n - 1]) | set(rng.integers(0, n, 40).tolist())))
    ra, rsfa = quant.quant_1x128(xa[rows])
    rb, rsfb = quant.quant_1x128(xb[cols])
    assert np.array_equal(host(a)[rows], ra) and np.array_equal(host(b)[cols], rb)
    ref = kgrouped.k_grouped_ref(ra, rsfa, rb, rsfb, offs)
    out = host(d)
    assert not np.any(out == SENTINEL)
    for grp in range(g):
        sub = out[grp][np.ix_(rows, cols)]
        if tokens[grp] == 0:
            assert np.all(out[grp] == 0)
        else:
            check(bf16_to_f64(sub), ref[grp], f"weight-gradient group {grp}")
