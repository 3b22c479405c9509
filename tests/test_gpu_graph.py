"""The entry points are graph-capturable (no allocation, no host sync, no
memset): a captured quantise + GEMM sequence, replayed several times with
eager work and synchronisations in between, must give the eager result bit
for bit on every replay.  Covered: the dense decode shape with stream-K K
parts (the arrival counters are reset inside the kernel, so the workspace
serves every replay), the masked layout whose valid-row counts change
between replays on the device, as in graph-captured MoE decode, and one
graph holding the contiguous layout with a quantised output (padding rows
included) and the K-grouped GEMM (an empty group included), and the UE8M0
column quantiser followed by the TN GEMM in K parts."""

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev, require_gpu

pytestmark = pytest.mark.gpu


def _bufs(dg, m, n, k, groups=None):
    shape_a = (m, k) if groups is None else (groups, m, k)
    shape_b = (n, k) if groups is None else (groups, n, k)
    x = dev(synth.bf16_normal(shape_a, 951))
    w = dev(synth.bf16_normal(shape_b, 952))
    a = torch.empty(shape_a, dtype=torch.uint8, device="cuda")
    ld = dg.dg_get_sf_leading_dim(m)
    sfa = torch.empty(((groups,) if groups else ()) + (k // 128, ld), dtype=torch.float32, device="cuda")
    b = torch.empty(shape_b, dtype=torch.uint8, device="cuda")
    sfb = torch.empty(((groups,) if groups else ()) + ((n + 127) // 128, k // 128), dtype=torch.float32, device="cuda")
    dg.dg_quant_128x128(w, b, sfb)
    ws_bytes = dg.dg_get_workspace_size(m, n, k, groups or 1)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    return x, a, sfa, b, sfb, ws


@pytest.mark.parametrize("m,n,k", [(128, 7168, 16384),   # 4 K parts per 128x128 tile
                                   (128, 4096, 7168)])   # 4 K parts per 64x64 tile, two workgroups per CU
def test_dense_stream_k_graph_replays(m, n, k):
    dg = require_gpu()
    cfg = dict(kv.split("=") for kv in dg.dg_describe_config(0, m, n, k, 1, dg.dg_get_num_cus()).split())
    assert int(cfg["stream_k"]) == 1
    x, a, sfa, b, sfb, ws = _bufs(dg, m, n, k)
    d = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

    def step():
        dg.dg_quant_1x128(x, a, sfa)
        dg.dg_fp8_gemm_nt(a, sfa, b, sfb, d, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = d.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        d.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_masked_graph_replays_with_changing_counts():
    dg = require_gpu()
    groups, m_max, n, k = 4, 256, 2048, 1536
    x, a, sfa, b, sfb, ws = _bufs(dg, m_max, n, k, groups)
    d = torch.empty((groups, m_max, n), dtype=torch.bfloat16, device="cuda")
    mm = torch.zeros(groups, dtype=torch.int32, device="cuda")

    def step():
        dg.dg_quant_1x128(x, a, sfa)
        dg.dg_grouped_masked(a, sfa, b, sfb, d, mm, expected_m=64, workspace=ws)

    counts = [np.array(c, dtype=np.int32) for c in ([64, 0, 200, 256], [1, 129, 77, 0], [256, 256, 256, 256])]
    eager = []
    for c in counts:
        mm.copy_(torch.from_numpy(c))
        d.fill_(0)
        step()
        torch.cuda.synchronize()
        eager.append(d.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(2):
        for c, want in zip(counts, eager):
            mm.copy_(torch.from_numpy(c))
            d.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(d.view(torch.int16), want.view(torch.int16)), f"counts {c.tolist()} pass {rep}"


def test_contiguous_qout_and_k_grouped_graph_replays():
    dg = require_gpu()
    # Contiguous with a quantised output: 4 row blocks of 128 owned by groups
    # 2, 0, padding (-1) and 3 of 4 experts.
    groups, m_total, n, k = 4, 512, 1024, 1024
    x = dev(synth.bf16_normal((m_total, k), 961))
    w = dev(synth.bf16_normal((groups, n, k), 962))
    a = torch.empty((m_total, k), dtype=torch.uint8, device="cuda")
    sfa = torch.empty((k // 128, dg.dg_get_sf_leading_dim(m_total)), dtype=torch.float32, device="cuda")
    b = torch.empty((groups, n, k), dtype=torch.uint8, device="cuda")
    sfb = torch.empty((groups, n // 128, k // 128), dtype=torch.float32, device="cuda")
    dg.dg_quant_128x128(w, b, sfb)
    ids = torch.from_numpy(np.repeat(np.array([2, 0, -1, 3], dtype=np.int32), 128)).cuda()
    d = torch.empty((m_total, n), dtype=torch.bfloat16, device="cuda")
    dq = torch.empty((m_total, n), dtype=torch.uint8, device="cuda")
    dsf = torch.empty((n // 128, dg.dg_get_sf_leading_dim(m_total)), dtype=torch.float32, device="cuda")
    # K-grouped: 3 groups over K = 2048 with offsets 0, 512, 512, 2048.
    m2, n2, k2 = 256, 512, 2048
    x2 = dev(synth.bf16_normal((m2, k2), 963))
    y2 = dev(synth.bf16_normal((n2, k2), 964))
    a2 = torch.empty((m2, k2), dtype=torch.uint8, device="cuda")
    sfa2 = torch.empty((k2 // 128, dg.dg_get_sf_leading_dim(m2)), dtype=torch.float32, device="cuda")
    b2 = torch.empty((n2, k2), dtype=torch.uint8, device="cuda")
    sfb2 = torch.empty((k2 // 128, dg.dg_get_sf_leading_dim(n2)), dtype=torch.float32, device="cuda")
    offs = torch.tensor([0, 512, 512, 2048], dtype=torch.int32, device="cuda")
    d2 = torch.empty((3, m2, n2), dtype=torch.bfloat16, device="cuda")
    outs = (d, dq, dsf, d2)

    def step():
        dg.dg_quant_1x128(x, a, sfa)
        dg.dg_grouped_contiguous_qout(a, sfa, b, sfb, d, dq, dsf, ids)
        dg.dg_quant_1x128(x2, a2, sfa2)
        dg.dg_quant_1x128(y2, b2, sfb2)
        dg.dg_k_grouped_nt(a2, sfa2, b2, sfb2, d2, offs)

    def clear():
        for t in outs:
            t.view(torch.uint8).fill_(0)

    clear()
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, want in zip(("d", "dq", "dsf", "d2"), outs, eager):
            assert torch.equal(t.view(torch.uint8), want.view(torch.uint8)), f"{name} differs on replay {r}"
        step()  # eager work between replays
        torch.cuda.synchronize()
    # The padding block stays untouched and the empty K group is zero.
    assert not torch.any(d[256:384].view(torch.int16)) and not torch.any(dq[256:384])
    assert not torch.any(d2[1].view(torch.int16))


def test_tn_ue8m0_graph_replays():
    """M-major activations quantised with exponent-byte scales by the column
    quantiser, then the TN GEMM in K parts (decode shape), in one graph."""
    dg = require_gpu()
    m, n, k = 128, 4096, 7168
    cfg = dict(kv.split("=") for kv in dg.dg_describe_config(0, m, n, k, 1, dg.dg_get_num_cus()).split())
    assert int(cfg["stream_k"]) == 1
    x_t = dev(synth.bf16_normal((k, m), 971))          # activations stored [K][M]
    w = dev(synth.bf16_normal((n, k), 972))
    a_t = torch.empty((k, m), dtype=torch.uint8, device="cuda")
    ea = torch.empty((k // 128, dg.dg_get_sf_leading_dim(m)), dtype=torch.uint8, device="cuda")
    b = torch.empty((n, k), dtype=torch.uint8, device="cuda")
    eb = torch.empty((k // 128, dg.dg_get_ue8m0_sfb_leading_dim(n)), dtype=torch.uint8, device="cuda")
    dg.dg_quant_128x128_ue8m0(w, b, eb)
    b_t = b.t().contiguous()                           # weights stored [K][N]
    ws_bytes = dg.dg_get_workspace_size(m, n, k, 1)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    d = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

    def step():
        dg.dg_quant_1x128_mn_ue8m0(x_t, a_t, ea)
        dg.dg_fp8_gemm_tn_ue8m0(a_t, ea, b_t, eb, d, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = d.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        d.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        step()
        torch.cuda.synchronize()
