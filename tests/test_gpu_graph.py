"""The entry points are graph-capturable (no allocation, no host sync, no
memset): a captured quantise + GEMM sequence, replayed several times with
eager work and synchronisations in between, must give the eager result bit
for bit on every replay.  Covered: the dense decode shape with stream-K K
parts (the arrival counters are reset inside the kernel, so the workspace
serves every replay), and the masked layout whose valid-row counts change
between replays on the device, as in graph-captured MoE decode."""

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
