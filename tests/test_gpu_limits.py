"""Operands at the size limit of the kernels' 32-bit byte offsets, and the
quantisers at the largest grids the host accepts.

Each e4m3 operand (per group) must stay below 4 GiB; the host rejects larger
ones.  These tests run operands just under that limit, so the last rows of A
or B (or the last K rows of an M-major A) sit at byte offsets near 2^32, and
check outputs that read them against the oracle: the first and last rows and
columns plus a few in between.

Inputs: random non-NaN e4m3 codes and fp32 scales drawn on the device with
seeded torch generators (no arithmetic of the method involved), copied back
for the oracle's sampled rows and columns.
"""

import numpy as np
import pytest
import torch

from oracle import majors, quant
from tests.gpu_util import SENTINEL, bf16_to_f64, host, require_gpu
from tests.tolerance import check

pytestmark = pytest.mark.gpu


def _codes(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    c = torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=g)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return c


def _scales(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.rand(shape, device="cuda", generator=g) * 1.5 + 0.5) * 2.0 ** -8


def _ws(dg, m, n, k):
    size = dg.dg_get_workspace_size(m, n, k, 1)
    return torch.zeros(size, dtype=torch.uint8, device="cuda") if size else None


def _sample(n_max, extra, seed):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set([0, 1, n_max - 2, n_max - 1]) | set(rng.integers(0, n_max, extra).tolist())))


def test_activation_just_under_4gib():
    """A [4096][1048448] (4294443008 bytes), N = 128: rows up to 4095 of A."""
    dg = require_gpu()
    m, n, k = 4096, 128, 1048448
    assert m * k < 2 ** 32 and (m + 1) * k > 2 ** 32 - 2 ** 21
    a = _codes((m, k), 2101)
    b = _codes((n, k), 2102)
    sfa = _scales((k // 128, m), 2103)
    sfb = _scales((1, k // 128), 2104)
    d = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt(a, sfa, b, sfb, d, workspace=_ws(dg, m, n, k))
    torch.cuda.synchronize()
    rows = _sample(m, 4, 2105)
    idx = torch.from_numpy(rows).cuda()
    a_rows = host(a.index_select(0, idx))
    sa_rows = np.ascontiguousarray(host(sfa.index_select(1, idx)))
    del a
    torch.cuda.empty_cache()
    ref = majors.gemm_layout_ref("nt", a_rows, sa_rows, host(b), host(sfb))
    check(bf16_to_f64(host(d)[rows]), ref, "A just under 4 GiB")


def test_weight_just_under_4gib():
    """B [32768][130944] (4290772992 bytes), M = 64: columns up to 32767."""
    dg = require_gpu()
    m, n, k = 64, 32768, 130944
    assert n * k < 2 ** 32
    a = _codes((m, k), 2111)
    b = _codes((n, k), 2112)
    sfa = _scales((k // 128, m), 2113)
    sfb = _scales((n // 128, k // 128), 2114)
    d = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt(a, sfa, b, sfb, d, workspace=_ws(dg, m, n, k))
    torch.cuda.synchronize()
    cols = _sample(n, 12, 2115)
    b_h = host(b.index_select(0, torch.from_numpy(cols).cuda()))
    sfb_h = host(sfb)
    del b
    torch.cuda.empty_cache()
    a_h, sfa_h = host(a), host(sfa)
    ref = np.stack([majors.gemm_layout_ref("nt", a_h, sfa_h, b_h[[i]], sfb_h[[c // 128]])[:, 0]
                    for i, c in enumerate(cols)], axis=1)
    check(bf16_to_f64(host(d)[:, cols]), ref, "B just under 4 GiB")


def test_m_major_activation_just_under_4gib():
    """TN: A stored [1048448][4096] (K rows of M bytes), B stored [K][128]:
    the last K rows of A sit near byte offset 2^32."""
    dg = require_gpu()
    m, n, k = 4096, 128, 1048448
    a_s = _codes((k, m), 2121)
    b_s = _codes((k, n), 2122)
    sfa = _scales((k // 128, m), 2123)
    sfb = _scales((1, k // 128), 2124)
    d = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_tn(a_s, sfa, b_s, sfb, d, workspace=_ws(dg, m, n, k))
    torch.cuda.synchronize()
    rows = _sample(m, 4, 2125)
    idx = torch.from_numpy(rows).cuda()
    a_cols = host(a_s.index_select(1, idx))  # [K][rows]: the sampled rows of the logical A
    sa_rows = np.ascontiguousarray(host(sfa.index_select(1, idx)))
    del a_s
    torch.cuda.empty_cache()
    ref = majors.gemm_layout_ref("tn", a_cols, sa_rows, host(b_s), host(sfb))
    check(bf16_to_f64(host(d)[rows]), ref, "M-major A just under 4 GiB")


def _bf16_normal(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)


def test_weight_quantiser_at_the_block_limit():
    """128x128 blocks: 65535 row blocks (the host's limit), the last one half
    full; sampled blocks, the first and last included, bit for bit."""
    dg = require_gpu()
    rows, cols = 65535 * 128 - 64, 128
    w = _bf16_normal((rows, cols), 2301)
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    sf = torch.full((65535, 1), float("nan"), dtype=torch.float32, device="cuda")
    dg.dg_quant_128x128(w, q, sf)
    torch.cuda.synchronize()
    sf_h = host(sf)
    for blk in _sample(65535, 6, 2302):
        r0, r1 = 128 * blk, min(128 * blk + 128, rows)
        rq, rsf = quant.quant_128x128(host(w[r0:r1]))
        assert np.array_equal(host(q[r0:r1]), rq), f"codes of block {blk}"
        assert sf_h[blk, 0].view(np.uint32) == rsf[0, 0].view(np.uint32), f"scale of block {blk}"


def test_column_quantiser_at_the_k_block_limit():
    """M-major activations with K = 65535 x 128 (the host's limit on K
    blocks), M = 8: sampled K blocks, the first and last included, bit for bit."""
    dg = require_gpu()
    k, m = 65535 * 128, 8
    x = _bf16_normal((k, m), 2311)
    q = torch.empty((k, m), dtype=torch.uint8, device="cuda")
    ld = dg.dg_get_sf_leading_dim(m)
    sf = torch.full((k // 128, ld), float("nan"), dtype=torch.float32, device="cuda")
    dg.dg_quant_1x128_mn(x, q, sf)
    torch.cuda.synchronize()
    sf_h = host(sf)
    for kb in _sample(k // 128, 6, 2312):
        rq, rsf = majors.quant_1x128_mn(host(x[128 * kb:128 * kb + 128]), ld_sf=ld)
        assert np.array_equal(host(q[128 * kb:128 * kb + 128]), rq), f"codes of K block {kb}"
        assert np.array_equal(sf_h[kb].view(np.uint32), rsf[0].view(np.uint32)), f"scales of K block {kb}"
