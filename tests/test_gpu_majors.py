"""GPU parity of the dense GEMM in the NN, TN and TT operand majors
(dg_fp8_gemm_nn / _tn / _tt) and of the column-wise activation quantiser
(dg_quant_1x128_mn), against oracle/majors.py.

An MN-major operand reaches the matrix cores through transposing LDS loads
that hand every lane the same K bytes, in the same order, as the K-major
path does; so for one tile configuration each layout must reproduce
dg_fp8_gemm_nt on the logical operands bit for bit.  Besides that the
outputs meet the bf16 tolerance rule against the oracle, equal the
oracle's rounding bit for bit on exact-grid inputs (every scale 2^-8, the
fp32 result exact in any order), and leave unwritten rows and columns alone.
The same holds with UE8M0 scales against dg_fp8_gemm_nt_ue8m0, and the
column quantisers (fp32 and UE8M0 scales) match the oracle bit for bit.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import bf16, majors, quant, ue8m0
from tests.gpu_util import SENTINEL, bf16_to_f64, dev, host, require_gpu
from tests.tolerance import check

pytestmark = pytest.mark.gpu

LAYOUTS = ["nn", "tn", "tt"]
VARIANTS = [0, 4, 5, 6]


def _stored(layout, a, b):
    a_s = a if layout[0] == "n" else np.ascontiguousarray(a.T)
    b_s = b if layout[1] == "t" else np.ascontiguousarray(b.T)
    return a_s, b_s


def _ws(dg, m, n, k):
    size = dg.dg_get_workspace_size(m, n, k, 1)
    return torch.zeros(size, dtype=torch.uint8, device="cuda") if size else None


def _run(dg, layout, a_s, sfa, b_s, sfb, m, n, k, ldd=None):
    full = torch.full((m, ldd or n), SENTINEL, dtype=torch.int16, device="cuda")
    fn = getattr(dg, f"dg_fp8_gemm_{layout}")
    a_t = a_s if isinstance(a_s, torch.Tensor) else dev(a_s)
    b_t = b_s if isinstance(b_s, torch.Tensor) else dev(b_s)
    fn(a_t, dev(sfa), b_t, dev(sfb), full[:, :n], workspace=_ws(dg, m, n, k))
    return host(full)


def _operands(m, n, k, seed, grid=False):
    gen = synth.bf16_grid if grid else synth.bf16_normal
    a, sfa = quant.quant_1x128(gen((m, k), seed))
    b, sfb = quant.quant_128x128(gen((n, k), seed + 1))
    return a, sfa, b, sfb


@pytest.fixture
def force(monkeypatch):
    def _set(variant, division=0, rotate=None):
        cfg = f"{variant}:{division}" + (f":{rotate}" if rotate is not None else "")
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    yield _set
    monkeypatch.delenv("DG_FORCE_CONFIG", raising=False)


SHAPES = [(16, 16, 128), (160, 272, 1536), (64, 2112, 7168), (128, 256, 16384), (512, 512, 512)]


@pytest.mark.parametrize("m,n,k", SHAPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_default_config(layout, m, n, k):
    dg = require_gpu()
    a, sfa, b, sfb = _operands(m, n, k, 1200 + m + n)
    a_s, b_s = _stored(layout, a, b)
    out = _run(dg, layout, a_s, sfa, b_s, sfb, m, n, k)
    check(bf16_to_f64(out), majors.gemm_layout_ref(layout, a_s, sfa, b_s, sfb), f"{layout} {m}x{n}x{k}")
    nt = _run(dg, "nt", a, sfa, b, sfb, m, n, k)
    assert np.array_equal(out, nt), f"{layout} {m}x{n}x{k}: differs from the NT result"


@pytest.mark.parametrize("division", [0, 1, 3])
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_every_variant(layout, variant, division, force):
    dg = require_gpu()
    force(variant, division)
    m, n, k = 160, 272, 1536
    a, sfa, b, sfb = _operands(m, n, k, 1301)
    a_s, b_s = _stored(layout, a, b)
    out = _run(dg, layout, a_s, sfa, b_s, sfb, m, n, k)
    check(bf16_to_f64(out), majors.gemm_layout_ref(layout, a_s, sfa, b_s, sfb), f"{layout} v{variant} d{division}")
    assert np.array_equal(out, _run(dg, "nt", a, sfa, b, sfb, m, n, k))


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_exact_grid_bitwise(layout, variant, force):
    dg = require_gpu()
    force(variant, 0)
    m, n, k = 208, 400, 1024
    a, sfa, b, sfb = _operands(m, n, k, 1401, grid=True)
    a_s, b_s = _stored(layout, a, b)
    ref = majors.gemm_layout_ref(layout, a_s, sfa, b_s, sfb)
    assert np.all(ref * 16 == np.round(ref * 16)) and np.abs(ref).max() < 2.0 ** 19
    out = _run(dg, layout, a_s, sfa, b_s, sfb, m, n, k)
    assert np.array_equal(out, bf16.bits_from_f64(ref))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_padded_leading_dims(layout):
    """Operands inside wider buffers (lda > m or k, ldb > n or k) and a padded
    output: padding columns of d stay untouched."""
    dg = require_gpu()
    m, n, k = 96, 144, 512
    a, sfa, b, sfb = _operands(m, n, k, 1501)
    a_s, b_s = _stored(layout, a, b)
    a_big = torch.zeros((a_s.shape[0], a_s.shape[1] + 48), dtype=torch.uint8, device="cuda")
    b_big = torch.zeros((b_s.shape[0], b_s.shape[1] + 32), dtype=torch.uint8, device="cuda")
    a_big[:, :a_s.shape[1]] = dev(a_s)
    b_big[:, :b_s.shape[1]] = dev(b_s)
    out = _run(dg, layout, a_big[:, :a_s.shape[1]], sfa, b_big[:, :b_s.shape[1]], sfb, m, n, k, ldd=n + 40)
    assert np.all(out[:, n:] == SENTINEL)
    check(bf16_to_f64(out[:, :n]), majors.gemm_layout_ref(layout, a_s, sfa, b_s, sfb), f"{layout} padded")


def test_rejections(force):
    dg = require_gpu()
    m, n, k = 40, 64, 256
    a, sfa, b, sfb = _operands(m, n, k, 1601)
    a_s, b_s = _stored("tn", a, b)
    with pytest.raises(dg.DGError) as err:  # M-major A needs m % 16 == 0
        _run(dg, "tn", a_s, sfa, b_s, sfb, m, n, k)
    assert err.value.status == -2
    a, sfa, b, sfb = _operands(48, 72, k, 1602)
    a_s, b_s = _stored("nn", a, b)
    with pytest.raises(dg.DGError) as err:  # N-major B needs n % 16 == 0
        _run(dg, "nn", a_s, sfa, b_s, sfb, 48, 72, k)
    assert err.value.status == -2
    force(1, 0)  # a tile built without MN-major instances
    a, sfa, b, sfb = _operands(48, 64, k, 1603)
    a_s, b_s = _stored("tt", a, b)
    with pytest.raises(dg.DGError) as err:
        _run(dg, "tt", a_s, sfa, b_s, sfb, 48, 64, k)
    assert err.value.status == -2


@pytest.mark.parametrize("k,m,ld", [(384, 136, 140), (128, 8, 8), (1024, 4096, 4096)])
def test_column_quantiser_bitwise(k, m, ld):
    dg = require_gpu()
    x = synth.bf16_normal((k, m), 1700 + m)
    x[128:256 if k > 128 else 128, 5 % m] = 0  # an all-zero column tile
    x[0:128, 2] = 0x8000                        # a tile of -0 only
    q_ref, sf_ref = majors.quant_1x128_mn(x, ld)
    q = torch.full((k, m), 0x5A, dtype=torch.uint8, device="cuda")
    sf = torch.full((k // 128, ld), -3.25, dtype=torch.float32, device="cuda")
    dg.dg_quant_1x128_mn(dev(x), q, sf)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(sf).view(np.uint32), sf_ref.view(np.uint32))


def test_weight_gradient_shape_sampled():
    """TN at 4096 x 4096 x 7168 (both operands quantised down their columns on
    the GPU): sampled rows and columns against the oracle, and the whole
    output against NT on the transposed codes."""
    dg = require_gpu()
    rng = np.random.default_rng(1801)
    m, n, k = 4096, 4096, 7168
    xa = synth.bf16_normal((k, m), 1802)   # stored [K][M]
    xb = synth.bf16_normal((n, k), 1803)   # weights [N][K], quantised per 128x128 block
    a_s = torch.empty((k, m), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((k // 128, m), dtype=torch.float32, device="cuda")
    dg.dg_quant_1x128_mn(dev(xa), a_s, sfa)
    b = torch.empty((n, k), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((n // 128, k // 128), dtype=torch.float32, device="cuda")
    dg.dg_quant_128x128(dev(xb), b, sfb)
    b_s = b.t().contiguous()               # N-major storage of the same codes
    d = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_tn(a_s, sfa, b_s, sfb, d, workspace=_ws(dg, m, n, k))
    d_nt = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt(a_s.t().contiguous(), sfa, b, sfb, d_nt, workspace=_ws(dg, m, n, k))
    torch.cuda.synchronize()
    assert torch.equal(d, d_nt)
    rows = np.array(sorted(set([0, m - 1]) | set(rng.integers(0, m, 10).tolist())))
    cols = np.array(sorted(set([0, n - 1]) | set(rng.integers(0, n, 40).tolist())))
    a_rows = np.ascontiguousarray(host(a_s)[:, rows].T)
    qa, sa_rows = quant.quant_1x128(np.ascontiguousarray(xa[:, rows].T))
    assert np.array_equal(a_rows, qa)
    # One oracle call per sampled column, with that column's block of weight
    # scales as a one-row scale matrix.
    b_h, sfb_h = host(b), host(sfb)
    ref = np.stack([majors.gemm_layout_ref("nt", a_rows, sa_rows, b_h[[c]], sfb_h[[c // 128]])[:, 0] for c in cols],
                   axis=1)
    check(bf16_to_f64(host(d)[np.ix_(rows, cols)]), ref, "tn 4096x4096x7168 sampled")


# --------------------------------------------------------- UE8M0 scales --

UE_VARIANTS = [0, 4, 5, 6]


def _ue_operands(m, n, k, seed):
    a, ea = ue8m0.quant_1x128_ue8m0(synth.bf16_normal((m, k), seed))
    b, eb = ue8m0.quant_128x128_ue8m0(synth.bf16_normal((n, k), seed + 1))
    return a, ea, b, eb


def _run_ue(dg, layout, a_s, ea, b_s, eb, m, n, k):
    d = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
    getattr(dg, f"dg_fp8_gemm_{layout}_ue8m0")(dev(a_s), dev(ea), dev(b_s), dev(eb), d, workspace=_ws(dg, m, n, k))
    return host(d)


@pytest.mark.parametrize("division", [0, 3])
@pytest.mark.parametrize("variant", UE_VARIANTS)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_ue8m0_every_variant(layout, variant, division, force):
    """UE8M0 scales: the same bytes reach the block-scaled MFMA as in NT, so
    the output equals dg_fp8_gemm_nt_ue8m0's bit for bit; and the oracle,
    fed the powers of two the exponents stand for, within tolerance."""
    dg = require_gpu()
    force(variant, division)
    m, n, k = 160, 272, 1536
    a, ea, b, eb = _ue_operands(m, n, k, 1901)
    a_s, b_s = _stored(layout, a, b)
    out = _run_ue(dg, layout, a_s, ea, b_s, eb, m, n, k)
    ref = majors.gemm_layout_ref(layout, a_s, ue8m0.sfa_as_fp32(ea), b_s, ue8m0.sfb_as_fp32(eb, n))
    check(bf16_to_f64(out), ref, f"{layout} ue8m0 v{variant} d{division}")
    assert np.array_equal(out, _run_ue(dg, "nt", a, ea, b, eb, m, n, k))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_ue8m0_default_config_decode_and_prefill(layout):
    dg = require_gpu()
    for m, n, k in [(64, 2112, 7168), (512, 1024, 2048)]:
        a, ea, b, eb = _ue_operands(m, n, k, 1911 + m)
        a_s, b_s = _stored(layout, a, b)
        out = _run_ue(dg, layout, a_s, ea, b_s, eb, m, n, k)
        ref = majors.gemm_layout_ref(layout, a_s, ue8m0.sfa_as_fp32(ea), b_s, ue8m0.sfb_as_fp32(eb, n))
        check(bf16_to_f64(out), ref, f"{layout} ue8m0 {m}x{n}x{k}")
        assert np.array_equal(out, _run_ue(dg, "nt", a, ea, b, eb, m, n, k))


@pytest.mark.parametrize("k,m,ld", [(384, 136, 140), (1024, 4096, 4096)])
def test_ue8m0_column_quantiser_bitwise(k, m, ld):
    dg = require_gpu()
    x = synth.bf16_normal((k, m), 1921 + m)
    x[0:128, 3] = 0
    x[128:256, 7] = 0x8000
    q_ref, sf_ref = majors.quant_1x128_mn_ue8m0(x, ld)
    q = torch.full((k, m), 0x5A, dtype=torch.uint8, device="cuda")
    sf = torch.full((k // 128, ld), 0xA5, dtype=torch.uint8, device="cuda")
    dg.dg_quant_1x128_mn_ue8m0(dev(x), q, sf)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(sf), sf_ref)
