"""The benchmark's JSON line keeps its contract: one line on stdout with the
metric fields, a roofline object and (unless disabled) the oracle's CPU
baseline; and a request for more than one GPU is refused."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline"}
ROOFLINE_KEYS = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


def _run(args, timeout=240):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT)


@pytest.mark.gpu
def test_json_line_contract():
    r = _run(["--workload", "dense_m64_n2112_k7168", "--steps", "3", "--warmup", "1", "--cpu-seconds", "1",
              "--per-shape", "step"])
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [line for line in r.stdout.splitlines() if line.strip()]
    assert len(lines) == 1, "exactly one line on stdout"
    out = json.loads(lines[0])
    assert KEYS <= set(out)
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert out["config"]["workload"] == "dense_m64_n2112_k7168"
    roof = out["roofline"]
    assert ROOFLINE_KEYS <= set(roof)
    assert roof["bound"] in ("hbm", "mfma") and 0 < roof["frac"] < 1
    assert abs(roof["achieved"] / roof["peak"] - roof["frac"]) < 1e-3
    shape = out["per_shape"][0]
    assert len(out["per_shape"]) == 1 and shape["workload"] == "dense_m64_n2112_k7168"
    assert shape["gemm_us_rocprof_median"] is None or shape["gemm_us_source"] == "rocprofv3 median"
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"], timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_loop_probe_runs_every_mode():
    # The register-only loop probe (libdg_probe.so) behind bench.py
    # --probe-ceiling: every mode at one and two waves per SIMD writes finite
    # sums for every thread and a positive cycle and tick count per workgroup.
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "moe_grouped_gemm_02_amd", "libdg_probe.so"))
    lib.dg_probe_loop.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    for mode in (0, 1, 2):
        for waves in (4, 8):
            wgs = 8
            out = torch.full((wgs * waves * 64,), float("nan"), dtype=torch.float32, device="cuda")
            clk = torch.zeros(wgs * 2, dtype=torch.int64, device="cuda")
            rc = lib.dg_probe_loop(mode, waves, wgs, 20, out.data_ptr(), clk.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            assert rc == 0
            assert bool(torch.isfinite(out).all()) and bool((out > 0).all()), (mode, waves)
            assert bool((clk > 0).all()), (mode, waves)
