#!/usr/bin/env python3
"""Benchmark of the fine-grained-scaled FP8 GEMM path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input: for
every shape of the workload, quantise the bf16 activations per 1x128 tile
(dg_quant_1x128) and run the GEMM (dg_fp8_gemm_nt, or the grouped entry
points) on weights that were quantised per 128x128 block once, before timing
(weights are converted offline, once per weight).

The default step is the largest workload: the MoE grouped GEMM in the
contiguous layout, 4 experts x 8192 rows, N = 4096, K = 7168 (quantise the
32768 x 7168 activations, then dg_grouped_contiguous).  Beside the step, the
JSON line carries a per-shape record for every shape of the five workloads
(dense M = 64; the M = 128 decode and M = 4096 prefill sweeps over six (N, K)
pairs; contiguous; masked), each with both roofline fractions.

Per-shape GEMM times: the primary figure is the median kernel duration from
a rocprofv3 kernel trace (a child process: 10 warm-up launches, then 60
timed ones per shape); the secondary is the mean over event-bracketed
launches in this process.  `--workload decode128` times the decode sweep as
the step instead; `--workload all` adds the pages' other table rows and the
extra layouts to the per-shape records.

Throughput accounting (the pages' own, which reproduces every row of the
DeepGEMM performance tables, see tests/golden/):
    flops = 2 * M_valid * N * K
    bytes = M_valid * K + G * N * K + 2 * M_valid * N   (fp8 A, fp8 B, bf16 D)
Scale bytes are reported separately.

Caches: every weight matrix is rotated through enough copies that the set
touched per step exceeds twice the 256 MB Infinity Cache, so weights come
from HBM, not from the L2s or MALL.
"""

import argparse
import json
import math
import os
import platform
import subprocess
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (no sparsity)
MALL_BYTES = 256 << 20
METRIC = "FP8 TFLOPS and HBM GB/s per shape, % of MI355X FP8/HBM roofline"

# DeepGEMM performance tables (H800), TFLOPS per (layout, groups, m per group,
# n, k): DeepGEMM project introduction, section Performance, kept with their
# citation in tests/golden/deepgemm_perf_tables.csv.  Context only.
def _load_pages_tflops():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests", "golden", "deepgemm_perf_tables.csv")
    table = {}
    with open(path) as f:
        rows = [line for line in f if line.strip() and not line.startswith("#")]
    for line in rows[1:]:
        layout, groups, m, n, k, tflops = line.split(",")[:6]
        table[(layout, int(groups), int(m), int(n), int(k))] = float(tflops)
    return table


PAGES_TFLOPS = _load_pages_tflops()


def pages_key(wl):
    """The pages' table row of a workload, or None (random masked counts are not a row)."""
    if (wl.layout == "masked" and not wl.all_valid) or wl.extra.get("majors", "nt") != "nt":
        return None  # the tables hold NT GEMMs only
    key = (wl.layout, wl.groups, wl.m, wl.n, wl.k)
    return key if key in PAGES_TFLOPS else None


def algorithmic_flops(m_valid, n, k):
    return 2.0 * m_valid * n * k


def algorithmic_bytes(m_valid, n, k, groups=1):
    return float(m_valid * k + groups * n * k + 2 * m_valid * n)


def scale_bytes(m_valid, n, k, groups=1, scales="fp32"):
    per = 1 if scales == "ue8m0" else 4
    return float(per * m_valid * (k // 128) + per * groups * ((n + 127) // 128) * (k // 128))


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="headline",
                   help="headline (default: contiguous 4 x 8192 x 4096 x 7168) | decode128 | all | pages | "
                        "a workload name from synth")
    p.add_argument("--no-rocprof", action="store_true",
                   help="skip the rocprofv3 kernel-trace pass (per-shape medians)")
    p.add_argument("--per-shape", choices=("workloads", "step"), default="workloads",
                   help="per-shape records for every shape of the five workloads (default) or the step's only")
    p.add_argument("--trace-child", metavar="NAMES",
                   help="internal: launch the GEMMs of these comma-separated workloads for a kernel trace")
    p.add_argument("--trace-warmup", type=int, default=10)
    p.add_argument("--trace-reps", type=int, default=60)
    p.add_argument("--scales", choices=("fp32", "ue8m0"), default="fp32",
                   help="scale format: fp32 (default) or power-of-two exponent bytes (UE8M0)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work for the oracle sample")
    p.add_argument("--probe-ceiling", action="store_true",
                   help="run only the register-only loop probe (libdg_probe.so) and write "
                        "profiles/mfma_loop_ceiling_gfx950.md")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain device copy of known size (for counter calibration)")
    p.add_argument("--launches-only", metavar="WORKLOADS",
                   help="only quantise and launch these comma-separated workloads' GEMMs --reps times each, in "
                        "order, no timing (the program rocprofv3 --pmc runs for the counter summaries)")
    p.add_argument("--reps", type=int, default=5)
    p.add_argument("--write-mfma", metavar="PMC_CSV",
                   help="with --launches-only W: write profiles/gemm_kernel_W_mfma.txt from a counter pass "
                        "over the MFMA counters (see write_mfma)")
    p.add_argument("--write-stalls", nargs=2, metavar=("PMC_CSV_A", "PMC_CSV_B"),
                   help="with --launches-only W: write profiles/gemm_kernel_W_stalls.txt (wave-time breakdown) "
                        "from the two counter passes of STALL_COUNTERS (no GPU needed)")
    p.add_argument("--num-cus", type=int, default=256, help="CUs of the measured GPU, for --write-mfma / --write-stalls")
    p.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                   help="write the traffic summary for --launches-only's workload from four rocprofv3 "
                        "counter_collection.csv files (no GPU needed)")
    return p.parse_args(argv)


# --------------------------------------------------------------- workloads --

HEADLINE = "contiguous_g4_m8192_n4096_k7168"


def select_workloads(name):
    import synth
    wls = synth.workloads()
    extra = synth.pages_workloads() + synth.extra_workloads()
    if name == "headline":
        return [w for w in wls if w.name == HEADLINE]
    if name == "decode128":
        return [w for w in wls if w.layout == "dense" and w.m == 128]
    if name == "all":
        return wls + extra
    if name == "pages":  # every row of the pages' performance tables
        return [w for w in wls + extra if pages_key(w) is not None]
    pick = [w for w in wls + extra if w.name == name]
    if not pick:
        raise SystemExit(f"unknown workload {name}; choose from headline, decode128, all, pages, "
                         + ", ".join(w.name for w in wls + extra))
    return pick


class Prepared:
    """Device buffers for one workload shape, weights rotated for cache misses."""

    def __init__(self, dg, torch, wl, scales="fp32"):
        import synth
        self.wl = wl
        self.scales = scales
        ue = scales == "ue8m0"
        sf_dtype = torch.uint8 if ue else torch.float32
        g, n, k = wl.groups, wl.n, wl.k
        dev = "cuda"
        kg = wl.layout == "k_grouped"
        if kg and ue:
            raise SystemExit("the K-grouped GEMM takes fp32 scales only")
        # Operand majors of a dense workload: "nt" (default), "nn", "tn", "tt".
        self.majors = wl.extra.get("majors", "nt")
        a_mn, b_mn = self.majors[0] == "t", self.majors[1] == "n"
        if wl.layout in ("dense", "k_grouped"):
            self.m_rows, a_shape = wl.m, (wl.m, k)
        elif wl.layout == "contiguous":
            self.m_rows, a_shape = g * wl.m, (g * wl.m, k)
        else:
            self.m_rows, a_shape = wl.m, (g, wl.m, k)
        if a_mn:
            a_shape = (k, wl.m)  # stored [K][M]
        xa = synth.bf16_normal(a_shape, wl.seed_a)
        self.x = torch.from_numpy(xa.view(np.int16)).to(dev)
        self.a = torch.empty(a_shape, dtype=torch.uint8, device=dev)
        ld = dg.dg_get_sf_leading_dim(self.m_rows)
        self.sfa = torch.empty(((g,) if wl.layout == "masked" else ()) + (k // 128, ld), dtype=sf_dtype, device=dev)
        b_shape = (n, k) if wl.layout in ("dense", "k_grouped") else (g, n, k)
        xb = torch.from_numpy(synth.bf16_normal(b_shape, wl.seed_b).view(np.int16)).to(dev)
        qb = torch.empty(b_shape, dtype=torch.uint8, device=dev)
        if kg:  # both operands activation-like: 1x128 scales along K
            sfb = torch.empty((k // 128, dg.dg_get_sf_leading_dim(n)), dtype=torch.float32, device=dev)
            dg.dg_quant_1x128(xb, qb, sfb)
        else:
            sfb_shape = (k // 128, dg.dg_get_ue8m0_sfb_leading_dim(n)) if ue else ((n + 127) // 128, k // 128)
            sfb = torch.empty(((g,) if wl.layout != "dense" else ()) + sfb_shape, dtype=sf_dtype, device=dev)
            (dg.dg_quant_128x128_ue8m0 if ue else dg.dg_quant_128x128)(xb, qb, sfb)
        del xb
        if b_mn:
            qb = qb.t().contiguous()  # N-major storage of the same codes (set-up, not timed)
        set_bytes = qb.numel() + sfb.numel() * sfb.element_size()
        copies = max(1, math.ceil(2 * MALL_BYTES / set_bytes)) if set_bytes < 2 * MALL_BYTES else 1
        copies = min(copies, 64)
        self.b = [qb] + [qb.clone() for _ in range(copies - 1)]
        self.sfb = [sfb] + [sfb.clone() for _ in range(copies - 1)]
        self.d = torch.empty(((g,) if wl.layout in ("masked", "k_grouped") else ()) + (self.m_rows, n),
                             dtype=torch.int16, device=dev)
        self.mi = None
        self.mm = None
        self.koffs = None
        if wl.layout == "contiguous":
            self.mi = torch.from_numpy(synth.contiguous_m_indices([wl.m] * g)).to(dev)
            self.m_valid = g * wl.m
        elif wl.layout == "masked":
            mm = synth.workload_masked_m(wl)
            self.mm = torch.from_numpy(mm).to(dev)
            self.m_valid = int(mm.sum())
        else:
            self.m_valid = wl.m
        if kg:
            self.koffs = torch.from_numpy(synth.k_group_offsets(wl)).to(dev)
        ws = dg.dg_get_workspace_size(self.m_rows, n, k, g)
        self.ws = torch.zeros(ws, dtype=torch.uint8, device=dev) if ws else None
        self.flops = algorithmic_flops(self.m_valid, n, k)
        self.bytes = algorithmic_bytes(self.m_valid, n, k, g)
        if kg:  # A and B once, G output matrices
            self.bytes = float(wl.m * k + n * k + 2 * g * wl.m * n)
        self.sf_bytes = scale_bytes(self.m_valid, n, k, g, scales)
        layout_id = {"dense": 0, "contiguous": 1, "masked": 2, "k_grouped": 3}[wl.layout]
        self.expected_m = self.m_valid // g if wl.layout == "masked" else 0
        self.config = dg.dg_describe_config(layout_id, self.m_rows, n, k, g, dg.dg_get_num_cus(), self.expected_m)
        # One kernel instance per (tile variant, layout, stream-K or not): the
        # unit rocprofv3 reports durations for.
        fields = dict(kv.split("=") for kv in self.config.split())
        lay = wl.layout if self.majors == "nt" else f"{wl.layout}_{self.majors}"
        self.kernel_key = (f"gemm_kernel variant={fields['variant']} bm={fields['bm']} bn={fields['bn']} "
                           f"layout={lay} stream_k={fields['stream_k']} scales={scales}")
        sfx = "_ue8m0" if ue else ""
        self._quant_a = getattr(dg, ("dg_quant_1x128_mn" if a_mn else "dg_quant_1x128") + sfx)
        self._gemm = getattr(dg, {"dense": f"dg_fp8_gemm_{self.majors}", "contiguous": "dg_grouped_contiguous",
                                  "masked": "dg_grouped_masked", "k_grouped": "dg_k_grouped_nt"}[wl.layout] + sfx)

    def quant(self, dg):
        self._quant_a(self.x, self.a, self.sfa)

    def gemm(self, dg, r):
        b, sfb = self.b[r % len(self.b)], self.sfb[r % len(self.sfb)]
        if self.wl.layout == "dense":
            self._gemm(self.a, self.sfa, b, sfb, self.d, workspace=self.ws)
        elif self.wl.layout == "contiguous":
            self._gemm(self.a, self.sfa, b, sfb, self.d, self.mi, workspace=self.ws)
        elif self.wl.layout == "k_grouped":
            self._gemm(self.a, self.sfa, b, sfb, self.d, self.koffs)
        else:
            self._gemm(self.a, self.sfa, b, sfb, self.d, self.mm, expected_m=self.expected_m, workspace=self.ws)


# ------------------------------------------------------------------ timing --

class HipEvents:
    """HIP events created with hipEventDisableSystemFence, through the HIP
    runtime already loaded in this process (torch's).  Default events add a
    system-scope fence to every record (a few us per launch on this GPU);
    these timestamp kernels without it."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        self.lib = ctypes.CDLL(path)
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        if self.lib.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev

    def record(self, ev, stream_handle):
        if self.lib.hipEventRecord(ev, self.ct.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def _enqueue_ahead(torch, enqueue_fn):
    """Run enqueue_fn while the GPU is held by a sleep kernel.

    The host then queues all the timed work before the GPU starts on it, so
    kernel timings are device time, not host launch rate.  Returns the host
    seconds spent enqueueing and whether the sleep outlasted them.
    """
    sleep_cycles = int(2e8)
    torch.cuda.synchronize()
    probe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probe[0].record()
    torch.cuda._sleep(sleep_cycles)
    probe[1].record()
    t0 = time.perf_counter()
    enqueue_fn()
    host_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    sleep_s = probe[0].elapsed_time(probe[1]) * 1e-3
    return host_s, sleep_s > host_s


def time_steps(dg, torch, preps, steps, warmup, hip=None, instrument=None):
    """Time `steps` whole steps; the GEMM launches of the shapes in
    `instrument` (default: all) are bracketed by events.

    Returns (total ms for the steps, per-launch GEMM ms [steps][shapes], NaN
    for shapes not instrumented).  The step is timed with torch events; the
    GEMM launches with fence-free HIP events (HipEvents) on the same stream,
    recorded right before and after each launch.  Every event record costs
    the stream about 0.8 us, so the step whose time is the benchmark value
    brackets only the dominant kernel's launches.
    """
    hip = hip or HipEvents()
    instrument = set(range(len(preps))) if instrument is None else set(instrument)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for w in range(warmup):
        for p in preps:
            p.quant(dg)
            p.gemm(dg, w)
    torch.cuda.synchronize()
    ev = [[(hip.create(), hip.create()) if i in instrument else None for i in range(len(preps))]
          for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def enqueue():
        start.record(stream)
        for s in range(steps):
            for i, p in enumerate(preps):
                p.quant(dg)
                if ev[s][i]:
                    hip.record(ev[s][i][0], sh)
                p.gemm(dg, warmup + s)
                if ev[s][i]:
                    hip.record(ev[s][i][1], sh)
        end.record(stream)

    host_s, ahead = _enqueue_ahead(torch, enqueue)
    if not ahead:
        print(f"warning: host enqueue ({host_s * 1e3:.1f} ms) outlasted the GPU sleep; timings include host gaps",
              file=sys.stderr)
    total_ms = start.elapsed_time(end)
    gemm_ms = np.array([[hip.elapsed_ms(*e) if e else np.nan for e in row] for row in ev])  # [steps][shapes]
    for row in ev:
        for e in row:
            if e:
                hip.destroy(e[0])
                hip.destroy(e[1])
    return total_ms, gemm_ms


def time_quant(dg, torch, p, reps=20):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p.quant(dg)

    def enqueue():
        s.record()
        for _ in range(reps):
            p.quant(dg)
        e.record()

    _enqueue_ahead(torch, enqueue)
    return s.elapsed_time(e) / reps


# ------------------------------------------------------------ CPU baseline --

def cpu_baseline(wls, target_s, scales="fp32"):
    """The oracle, single-threaded, on a bounded sample of the workload.

    Sample, per shape: a 256-row slice of A (all rows when M <= 256; for the
    grouped layouts the first 256 rows of expert 0) against the whole of
    that expert's weight matrix when the step is a single large shape, or
    against its first 1024 columns (eight 128-row weight blocks) when the
    step is a sweep of shapes.  The activations are quantised inside the
    timed region, as in the GPU step; the weights are quantised before it.
    The sample is repeated until about target_s seconds of oracle work are
    done.  Rate = sample flops / oracle seconds; the oracle's cost is linear
    in the rows, so the whole step's oracle time is extrapolated from it and
    labelled as such.
    """
    import synth
    from oracle import gemm, quant, ue8m0
    from threadpoolctl import threadpool_limits

    if scales == "ue8m0":
        def quant_b(xb):
            qb, eb = ue8m0.quant_128x128_ue8m0(xb)
            return qb, ue8m0.sfb_as_fp32(eb, xb.shape[0])

        def quant_a(xa):
            qa, ea = ue8m0.quant_1x128_ue8m0(xa)
            return qa, ue8m0.sfa_as_fp32(ea)
    else:
        quant_b, quant_a = quant.quant_128x128, quant.quant_1x128

    whole_n = len(wls) == 1
    samples = []
    step_flops = 0.0
    for wl in wls:
        m = min(wl.m, 256)
        ncols = wl.n if whole_n else min(wl.n, 1024)
        rows_all = wl.m * wl.groups if wl.layout == "contiguous" else (
            int(synth.workload_masked_m(wl).sum()) if wl.layout == "masked" else wl.m)
        step_flops += algorithmic_flops(rows_all, wl.n, wl.k)
        # Expert 0's first rows and weights.  The generator fills tensors in
        # row-major order from one stream, so drawing only the leading rows
        # gives the same values as the full tensors' leading rows.
        xa = synth.bf16_normal((m, wl.k), wl.seed_a)
        xb = synth.bf16_normal((ncols, wl.k), wl.seed_b)
        qb, sfb = quant_b(xb)
        samples.append((wl, m, ncols, np.ascontiguousarray(xa), qb, sfb))
    flops = 0.0
    secs = 0.0
    runs = 0
    with threadpool_limits(limits=1):
        while secs < target_s and runs < 50 * len(samples):
            wl, m, ncols, xa, qb, sfb = samples[runs % len(samples)]
            t0 = time.perf_counter()
            qa, sfa = quant_a(xa)
            gemm.gemm_nt_ref(qa, sfa, qb, sfb)
            secs += time.perf_counter() - t0
            flops += algorithmic_flops(m, ncols, wl.k)
            runs += 1
    names = ", ".join(f"{wl.name}[rows :{m}, cols :{nc}]" for wl, m, nc, *_ in samples)
    rate = flops / secs
    return {
        "value": rate / 1e12,
        "unit": "TFLOPS",
        "cores": 1,
        "kind": "oracle",
        "sample": f"single-threaded numpy oracle (quantise A per 1x128 + fp64 blockwise GEMM) on a bounded slice: "
                  f"{names}; {runs} runs, {secs:.1f} s of CPU work",
        "extrapolated_step_s": round(step_flops / rate, 1),
        "extrapolation": "whole step's oracle time = step flops / sample rate (cost is linear in rows and columns)",
        "cpu_model": _cpu_model(),
        "host_cores": os.cpu_count(),
    }


# ------------------------------------------------------- rocprofv3 medians --

def trace_child(dg, torch, names, warmup, reps, scales):
    """Kernel-trace program: for each workload in turn, quantise once, then
    launch its GEMM warmup + reps times (weights rotated), synchronising
    between workloads.  Only GEMM launches are made after the set-up of each
    workload, so the parent can split the traced gemm_kernel dispatches into
    consecutive groups of warmup + reps."""
    import synth
    allw = {w.name: w for w in synth.workloads() + synth.pages_workloads() + synth.extra_workloads()}
    for name in names:
        p = Prepared(dg, torch, allw[name], scales)
        p.quant(dg)
        torch.cuda.synchronize()
        for r in range(warmup + reps):
            p.gemm(dg, r)
        torch.cuda.synchronize()
        print(json.dumps({"traced": name, "launches": warmup + reps}), flush=True)
        del p
        torch.cuda.empty_cache()


def _under_rocprof():
    return any("rocprof" in os.environ.get(v, "") for v in ("LD_PRELOAD", "HSA_TOOLS_LIB"))


def rocprof_medians(names, scales, warmup=10, reps=60, timeout_s=600):
    """Median kernel durations (us) per workload from a rocprofv3 kernel
    trace of a child process (trace_child), or None where unavailable."""
    import csv
    import glob
    import shutil
    import tempfile
    exe = shutil.which("rocprofv3")
    if exe is None or _under_rocprof():
        return None, "rocprofv3 not available" if exe is None else "already under rocprofv3"
    out = tempfile.mkdtemp(prefix="dg_trace_", dir=os.environ.get("TMPDIR", "/tmp"))
    cmd = [exe, "--kernel-trace", "--output-format", "csv", "-d", out, "-o", "kt", "--",
           sys.executable, os.path.abspath(__file__), "--trace-child", ",".join(names),
           "--trace-warmup", str(warmup), "--trace-reps", str(reps), "--scales", scales]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout_s, cwd=os.path.dirname(out))
    except subprocess.TimeoutExpired:
        shutil.rmtree(out, ignore_errors=True)
        return None, f"rocprofv3 child timed out after {timeout_s} s"
    done = [json.loads(x)["traced"] for x in r.stdout.splitlines() if x.startswith('{"traced"')]
    files = glob.glob(os.path.join(out, "**", "*kernel_trace.csv"), recursive=True)
    rows = []
    for path in files:
        with open(path) as f:
            for row in csv.DictReader(f):
                if "gemm_kernel" in row["Kernel_Name"]:
                    rows.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"])))
    shutil.rmtree(out, ignore_errors=True)
    rows.sort()
    per = warmup + reps
    if done != list(names) or len(rows) != per * len(names):
        return None, (f"rocprofv3 child incomplete (rc {r.returncode}, {len(done)}/{len(names)} workloads, "
                      f"{len(rows)} gemm dispatches)")
    med = {}
    for i, name in enumerate(names):
        durs = [(e - b) / 1e3 for b, e in rows[i * per + warmup:(i + 1) * per]]
        med[name] = float(np.median(durs))
    return med, f"rocprofv3 --kernel-trace: median of {reps} launches after {warmup} warm-up launches per shape"


def _cpu_model():
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# -------------------------------------------------------------------- main --

# ------------------------------------------------------------------ traffic --
#
# HBM traffic of the dominant kernel comes from two rocprofv3 --pmc runs of
# `bench.py --launches-only W` (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch) and the same two counters read for a plain 256 MiB device copy
# (`bench.py --calibrate-copy`), which scale them to bytes.  The summary is
# kept under profiles/ with a hash of the kernel sources; the bench line
# reports it only while the sources are unchanged.

PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
KERNEL_SOURCES = ("dg_gemm.hip", "dg_device.h", "dg_internal.h")
COPY_BYTES = 256 << 20


def _strip_comments(text):
    """C++ source without its // and /* */ comments and with runs of
    whitespace collapsed, so that editing a comment keeps the hash."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """Hash of the GEMM kernel sources' code (comments excluded): counter
    summaries taken from other code are not reported."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "moe_grouped_gemm_02_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(_strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def _counter_values(path, counter, name_part):
    """Per-dispatch values of one counter (summed over its instances) for the
    kernels whose name contains name_part, in dispatch order."""
    import csv
    sums = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                d = int(r["Dispatch_Id"])
                sums[d] = sums.get(d, 0.0) + float(r["Counter_Value"])
    if not sums:
        raise SystemExit(f"no {counter} rows for kernels matching {name_part!r} in {path}")
    return [sums[d] for d in sorted(sums)]


def _per_workload(values, workloads, reps, what):
    """Split dispatch-ordered values into the workloads' consecutive groups
    of `reps` launches (bench.py --launches-only W1,W2,... launches each
    workload's GEMM reps times, in order) and take each group's median."""
    if len(values) != reps * len(workloads):
        raise SystemExit(f"{what}: {len(values)} GEMM dispatches for {len(workloads)} workloads x {reps} launches")
    return [(float(np.median(values[i * reps:(i + 1) * reps])), reps) for i in range(len(workloads))]


def traffic_path(workload, scales="fp32"):
    return os.path.join(PROFILES, f"gemm_kernel_{workload}{'_ue8m0' if scales == 'ue8m0' else ''}_traffic.txt")


def _launch_cmd(workloads, scales, reps):
    sflag = " --scales ue8m0" if scales == "ue8m0" else ""
    return f"$REPO/bench.py --launches-only {','.join(workloads)} --reps {reps}{sflag}"


def write_traffic(workloads, scales, reps, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    fetch = _per_workload(_counter_values(fetch_csv, "FETCH_SIZE", "gemm_kernel"), workloads, reps, "FETCH_SIZE")
    write = _per_workload(_counter_values(write_csv, "WRITE_SIZE", "gemm_kernel"), workloads, reps, "WRITE_SIZE")
    cfetch = float(np.median(_counter_values(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")))
    cwrite = float(np.median(_counter_values(copy_write_csv, "WRITE_SIZE", "copyBuffer")))
    fscale, wscale = COPY_BYTES / (cfetch * 1024), COPY_BYTES / (cwrite * 1024)
    cmd = _launch_cmd(workloads, scales, reps)
    for wl, (f_kib, nf), (w_kib, nw) in zip(workloads, fetch, write):
        traffic = f_kib * 1024 * fscale + w_kib * 1024 * wscale
        lines = [
            f"workload={wl}",
            f"scales={scales}",
            f"kernel_source_sha256_16={kernel_source_hash()}",
            f"fetch_kib_per_dispatch={f_kib:.1f}  (median of {nf} dispatches)",
            f"write_kib_per_dispatch={w_kib:.1f}  (median of {nw} dispatches)",
            f"copy_fetch_kib={cfetch:.1f}  copy_write_kib={cwrite:.1f}  (plain copy of {COPY_BYTES} bytes each way)",
            f"fetch_scale={fscale:.4f}  write_scale={wscale:.4f}",
            f"traffic_bytes_per_launch={traffic:.0f}",
            "",
            "commands (from the repository root, REPO = its absolute path):",
            "  cd /tmp && export TMPDIR=/tmp",
            "  rocprofv3 --pmc FETCH_SIZE -f csv -d $REPO/gpurun_out/pmc_copy_f -o p -- python3 $REPO/bench.py --calibrate-copy",
            "  rocprofv3 --pmc WRITE_SIZE -f csv -d $REPO/gpurun_out/pmc_copy_w -o p -- python3 $REPO/bench.py --calibrate-copy",
            f"  rocprofv3 --pmc FETCH_SIZE -f csv -d $REPO/gpurun_out/pmc_f -o p -- python3 {cmd}",
            f"  rocprofv3 --pmc WRITE_SIZE -f csv -d $REPO/gpurun_out/pmc_w -o p -- python3 {cmd}",
            f"  python3 {cmd.replace('$REPO/', '')} --write-traffic gpurun_out/pmc_f/p_counter_collection.csv "
            "gpurun_out/pmc_w/p_counter_collection.csv gpurun_out/pmc_copy_f/p_counter_collection.csv "
            "gpurun_out/pmc_copy_w/p_counter_collection.csv",
        ]
        path = traffic_path(wl, scales)
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(path)


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_INSTS_MFMA "
                 "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")
MI355X_XCDS = 8


def mfma_path(workload, scales="fp32"):
    return os.path.join(PROFILES, f"gemm_kernel_{workload}{'_ue8m0' if scales == 'ue8m0' else ''}_mfma.txt")


def write_mfma(workloads, scales, reps, pmc_csv, num_cus):
    """MFMA-busy fraction of each workload's GEMM launches from one counter
    pass: SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (GRBM_GUI_ACTIVE per
    XCD x SIMDs), medians over the workload's dispatches; plus the MFMA op
    count against the algorithmic flops."""
    busy = _per_workload(_counter_values(pmc_csv, "SQ_VALU_MFMA_BUSY_CYCLES", "gemm_kernel"), workloads, reps, "busy")
    gui = _per_workload(_counter_values(pmc_csv, "GRBM_GUI_ACTIVE", "gemm_kernel"), workloads, reps, "gui")
    mops = _per_workload(_counter_values(pmc_csv, "SQ_INSTS_VALU_MFMA_MOPS_F8", "gemm_kernel"), workloads, reps, "mops")
    simds = 4 * num_cus
    cmd = _launch_cmd(workloads, scales, reps)
    for wl, (b, nd), (g, _), (mo, _) in zip(workloads, busy, gui, mops):
        frac = b / (g / MI355X_XCDS * simds)
        lines = [
            f"workload={wl}",
            f"scales={scales}",
            f"kernel_source_sha256_16={kernel_source_hash()}",
            f"mfma_busy_cycles={b:.6g}  (SQ_VALU_MFMA_BUSY_CYCLES, median of {nd} dispatches, all SIMDs)",
            f"grbm_gui_active={g:.6g}  (summed over {MI355X_XCDS} XCDs)",
            f"simds={simds}",
            f"mfma_busy_frac={frac:.4f}",
            f"mfma_flops={mo * 512:.6g}  (SQ_INSTS_VALU_MFMA_MOPS_F8 x 512)",
            "",
            "commands (from the repository root, REPO = its absolute path):",
            "  cd /tmp && export TMPDIR=/tmp",
            f"  rocprofv3 --pmc {MFMA_COUNTERS} -f csv -d $REPO/gpurun_out/pmcm -o p -- python3 {cmd}",
            f"  python3 {cmd.replace('$REPO/', '')} --write-mfma gpurun_out/pmcm/p_counter_collection.csv",
        ]
        path = mfma_path(wl, scales)
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(path)


# Where a GEMM's wave time goes: two rocprofv3 --pmc passes over
# `bench.py --launches-only W1,W2,...` (each within one pass's hardware
# limits: at most 8 SQ, 1 TA and 1 GRBM counter).
STALL_COUNTERS = (
    "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
    "SQ_INSTS_VALU SQ_INSTS_LDS GRBM_GUI_ACTIVE TA_TA_BUSY",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_SALU SQ_ACTIVE_INST_SCA SQ_LDS_CMD_FIFO_FULL "
    "SQ_LDS_DATA_FIFO_FULL SQ_WAVES GRBM_GUI_ACTIVE",
)


def stalls_path(workload, scales="fp32"):
    return os.path.join(PROFILES, f"gemm_kernel_{workload}{'_ue8m0' if scales == 'ue8m0' else ''}_stalls.txt")


def write_stalls(workloads, scales, reps, csv_a, csv_b, num_cus):
    """Wave-time breakdown of each workload's GEMM launches, medians over its
    dispatches.  SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_* count
    quad-cycles summed over all waves, so their ratios are shares of the
    waves' resident time: waiting at s_waitcnt or s_barrier (WAIT_ANY),
    ready but not issued (WAIT_INST_ANY: the SIMD's issue port, the matrix
    core or a dependency is busy), issuing VALU / LDS / scalar instructions.
    The busy fractions divide by GRBM_GUI_ACTIVE per XCD (the kernel's
    cycles) times the number of SIMDs, CUs or TA units."""
    def med(path, counter):
        return [v for v, _ in _per_workload(_counter_values(path, counter, "gemm_kernel"), workloads, reps, counter)]
    a = {c: med(csv_a, c) for c in STALL_COUNTERS[0].split()}
    b = {c: med(csv_b, c) for c in STALL_COUNTERS[1].split()}
    cmd = _launch_cmd(workloads, scales, reps)
    for i, wl in enumerate(workloads):
        cyc = a["GRBM_GUI_ACTIVE"][i] / MI355X_XCDS
        wave = a["SQ_WAVE_CYCLES"][i]
        mfma = b["SQ_INSTS_MFMA"][i]
        share = lambda c: a[c][i] / wave
        lines = [
            f"workload={wl}",
            f"scales={scales}",
            f"kernel_source_sha256_16={kernel_source_hash()}",
            f"kernel_cycles={cyc:.6g}  (GRBM_GUI_ACTIVE per XCD, median of {reps} dispatches)",
            f"waves={b['SQ_WAVES'][i]:.6g}",
            "shares of resident wave time (SQ_WAVE_CYCLES):",
            f"  wait_any={share('SQ_WAIT_ANY'):.3f}  (s_waitcnt / s_barrier: memory, LDS and barrier waits)",
            f"  wait_inst_any={share('SQ_WAIT_INST_ANY'):.3f}  (ready, not issued: issue port, matrix core or dependency busy)",
            f"  wait_inst_lds={share('SQ_WAIT_INST_LDS'):.3f}  (waiting to issue an LDS instruction)",
            f"  active_valu={share('SQ_ACTIVE_INST_VALU'):.3f}  (VALU and MFMA issue)",
            f"  active_lds={share('SQ_ACTIVE_INST_LDS'):.3f}",
            f"  active_sca={b['SQ_ACTIVE_INST_SCA'][i] / wave:.3f}  (scalar; second pass)",
            f"mfma_busy_frac={b['SQ_VALU_MFMA_BUSY_CYCLES'][i] / (b['GRBM_GUI_ACTIVE'][i] / MI355X_XCDS * 4 * num_cus):.4f}",
            f"ta_busy_frac={a['TA_TA_BUSY'][i] / (cyc * num_cus):.4f}  (address unit feeding the LDS DMA, per CU)",
            f"lds_cmd_fifo_full_frac={b['SQ_LDS_CMD_FIFO_FULL'][i] / (b['GRBM_GUI_ACTIVE'][i] / MI355X_XCDS * num_cus):.4f}"
            f"  lds_data_fifo_full_frac={b['SQ_LDS_DATA_FIFO_FULL'][i] / (b['GRBM_GUI_ACTIVE'][i] / MI355X_XCDS * num_cus):.4f}",
            f"mfma_insts={mfma:.6g}",
            f"valu_insts_per_mfma={(a['SQ_INSTS_VALU'][i] - mfma) / mfma:.2f}  (SQ_INSTS_VALU counts the MFMAs too)",
            f"lds_insts_per_mfma={a['SQ_INSTS_LDS'][i] / mfma:.2f}",
            f"salu_insts_per_mfma={b['SQ_INSTS_SALU'][i] / mfma:.2f}",
            "",
            "commands (from the repository root, REPO = its absolute path):",
            "  cd /tmp && export TMPDIR=/tmp",
            f"  rocprofv3 --pmc {STALL_COUNTERS[0]} -f csv -d $REPO/gpurun_out/pmcs_a -o p -- python3 {cmd}",
            f"  rocprofv3 --pmc {STALL_COUNTERS[1]} -f csv -d $REPO/gpurun_out/pmcs_b -o p -- python3 {cmd}",
            f"  python3 {cmd.replace('$REPO/', '')} --write-stalls gpurun_out/pmcs_a/p_counter_collection.csv "
            "gpurun_out/pmcs_b/p_counter_collection.csv",
        ]
        path = stalls_path(wl, scales)
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(path)


PROBE_MODES = (("mfma_chains", "16 accumulating MFMA chains per wave (C = acc)"),
               ("fp32_promotion", "per fragment row 4 MFMAs into partials, 1 scale multiply, 16 FMAs acc += P*s"),
               ("block_scaled", "32 block-scaled MFMAs accumulating in the matrix core (UE8M0 form)"))
FP8_FLOP_PER_CLK_PER_CU = 8192


def probe_ceiling(torch, workgroups=256, iters=2000, reps=5):
    """Run the register-only loop probe (libdg_probe.so, include/dg_probe.h)
    for each mode at one and two waves per SIMD; write
    profiles/mfma_loop_ceiling_gfx950.md and return its rows."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "moe_grouped_gemm_02_amd",
                                   "libdg_probe.so"))
    lib.dg_probe_loop.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.dg_probe_mfma_per_iter.argtypes = [ctypes.c_int]
    rows = []
    for mode, (name, what) in enumerate(PROBE_MODES):
        for waves in (4, 8):
            out = torch.empty(workgroups * waves * 64, dtype=torch.float32, device="cuda")
            clk = torch.zeros(workgroups * 2, dtype=torch.int64, device="cuda")
            stream = torch.cuda.current_stream()
            times = []
            for r in range(2 + reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                rc = lib.dg_probe_loop(mode, waves, workgroups, iters, ctypes.c_void_p(out.data_ptr()),
                                       ctypes.c_void_p(clk.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
                e1.record(stream)
                if rc != 0:
                    raise RuntimeError(f"dg_probe_loop returned {rc}")
                torch.cuda.synchronize()
                if r >= 2:
                    times.append(e0.elapsed_time(e1) * 1e-3)
            if not bool(torch.isfinite(out).all()):
                raise RuntimeError("probe accumulators not finite")
            c = clk.view(-1, 2).double().cpu()
            ghz = float(np.median((c[:, 0] / (c[:, 1] / 100e6)).numpy())) / 1e9
            flops = workgroups * waves * iters * lib.dg_probe_mfma_per_iter(mode) * 2 * 16 * 16 * 128
            t = float(np.median(times))
            pf = flops / t / 1e15
            at_clock = flops / t / (workgroups * FP8_FLOP_PER_CLK_PER_CU * ghz * 1e9)
            rows.append({"mode": name, "what": what, "waves_per_simd": waves // 4, "pflops": round(pf, 3),
                         "frac_of_5p0": round(pf / 5.0, 3), "clock_ghz": round(ghz, 3),
                         "frac_at_measured_clock": round(at_clock, 3), "ms": round(t * 1e3, 3)})
            print(json.dumps(rows[-1]), flush=True)
    lines = [
        "# Register-only loop ceilings on MI355X (gfx950): the GEMM inner loop's instruction mixes",
        "",
        "Command (from the repository root): `python3 bench.py --probe-ceiling`",
        "",
        f"Kernel: `probe_kernel<MODE>` of `moe_grouped_gemm_02_amd/csrc/dg_probe.hip` (libdg_probe.so), "
        f"{workgroups} workgroups (one per CU), {iters} iterations; every operand in registers, no LDS or global "
        "memory inside the timed loop. Time: median of "
        f"{reps} launches (torch events, after 2 warm-up launches). Clock: median over workgroups of s_memtime "
        "cycles / s_memrealtime (100 MHz) ticks over the loop. `frac_of_5p0` divides by the 5.0 PFLOP/s dense "
        "FP8 peak (2.4 GHz); `frac_at_measured_clock` by 256 CUs x 8192 flop/clk x the measured clock.",
        "",
        "| mode | loop | waves per SIMD | PFLOP/s | of 5.0 PF | clock GHz | of peak at that clock |",
        "|---|---|---:|---:|---:|---:|---:|",
    ]
    for r in rows:
        lines.append(f"| {r['mode']} | {r['what']} | {r['waves_per_simd']} | {r['pflops']} | {r['frac_of_5p0']} | "
                     f"{r['clock_ghz']} | {r['frac_at_measured_clock']} |")
    with open(os.path.join(PROFILES, "mfma_loop_ceiling_gfx950.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return rows


def _read_summary(path, key):
    """A value from a committed counter summary, or None if there is none or
    the kernel sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith(" "):
                k, v = line.split("=", 1)
                fields[k.strip()] = v.split()[0]
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return float(fields[key])


def read_mfma_busy(workload, scales="fp32"):
    return _read_summary(mfma_path(workload, scales), "mfma_busy_frac")


def read_traffic(workload, scales="fp32"):
    """Bytes per launch from the committed summary, or None if there is none
    for this workload or the kernel sources changed since it was taken."""
    return _read_summary(traffic_path(workload, scales), "traffic_bytes_per_launch")


def main(argv=None):
    args = parse_args(argv)
    if args.write_traffic:
        if not args.launches_only:
            raise SystemExit("--write-traffic needs --launches-only WORKLOADS")
        write_traffic(args.launches_only.split(","), args.scales, args.reps, *args.write_traffic)
        return 0
    if args.write_stalls:
        if not args.launches_only:
            raise SystemExit("--write-stalls needs --launches-only WORKLOADS")
        write_stalls(args.launches_only.split(","), args.scales, args.reps, *args.write_stalls, args.num_cus)
        return 0
    if args.write_mfma:
        if not args.launches_only:
            raise SystemExit("--write-mfma needs --launches-only WORKLOADS")
        write_mfma(args.launches_only.split(","), args.scales, args.reps, args.write_mfma, args.num_cus)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.probe_ceiling:
        probe_ceiling(torch)
        return 0
    import moe_grouped_gemm_02_amd as dg

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel(), "launches": 5}))
        return 0

    if args.launches_only:
        import synth
        allw = {w.name: w for w in synth.workloads() + synth.pages_workloads() + synth.extra_workloads()}
        for name in args.launches_only.split(","):
            p = Prepared(dg, torch, allw[name], args.scales)
            for r in range(args.reps):
                p.quant(dg)
                p.gemm(dg, r)
            torch.cuda.synchronize()
            print(json.dumps({"launches": args.reps, "workload": name, "config": p.config}), flush=True)
            del p
            torch.cuda.empty_cache()
        return 0

    if args.trace_child:
        trace_child(dg, torch, args.trace_child.split(","), args.trace_warmup, args.trace_reps, args.scales)
        return 0

    import synth
    wls = select_workloads(args.workload)
    headline = ([w for w in wls if w.layout == "dense" and w.m == 128] if args.workload == "decode128" else wls[:1])
    # Per-shape records: every shape of the five workloads, plus (for
    # --workload all / pages) the other shapes selected.
    shape_wls = list(synth.workloads()) if args.per_shape == "workloads" else []
    if args.workload in ("all", "pages"):
        shape_wls += [w for w in wls if w not in shape_wls]
    for w in headline:
        if w not in shape_wls:
            shape_wls.append(w)

    # rocprofv3 kernel-trace medians (primary per-shape times), taken in a
    # child process before this one touches the GPU.
    medians, median_note = (None, "skipped (--no-rocprof)") if args.no_rocprof else rocprof_medians(
        [w.name for w in shape_wls], args.scales)
    if medians is None:
        print(f"note: no rocprofv3 medians: {median_note}", file=sys.stderr)

    preps = [Prepared(dg, torch, w, args.scales) for w in headline]
    torch.cuda.synchronize()
    # Per-launch pass (not the benchmark value): every GEMM launch bracketed
    # by events, which also picks the dominant kernel - the GEMM
    # configuration with the most total time.
    _, shape_ms = time_steps(dg, torch, preps, args.steps, args.warmup)
    by_kernel = {}
    for i, p in enumerate(preps):
        by_kernel.setdefault(p.kernel_key, []).append(i)
    key = max(by_kernel, key=lambda k_: sum(float(np.sum(shape_ms[:, i])) for i in by_kernel[k_]))
    idx = by_kernel[key]

    # The timed pass: W warmup steps, then exactly K steps between two torch
    # events; only the dominant kernel's launches carry HIP events (each
    # event record costs the stream ~0.8 us).
    total_ms, gemm_ms = time_steps(dg, torch, preps, args.steps, args.warmup, instrument=idx)
    ms_per_step = total_ms / args.steps
    step_flops = sum(p.flops for p in preps)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    head_quant_ms = [time_quant(dg, torch, p) for p in preps]
    head_shape_ms = {p.wl.name: float(np.mean(shape_ms[:, i])) for i, p in enumerate(preps)}

    # Roofline of the dominant kernel, from its launches in the timed pass.
    # HBM-bound below the ridge point (peak flops / peak bytes), MFMA-bound
    # above it.
    mean_bytes = float(np.mean([preps[i].bytes for i in idx]))
    mean_flops = float(np.mean([preps[i].flops for i in idx]))
    mean_dur = float(np.mean(gemm_ms[:, idx])) * 1e-3
    mfma_bound = mean_flops / mean_bytes > FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    achieved = mean_flops / mean_dur / 1e12 if mfma_bound else mean_bytes / mean_dur / 1e9
    peak = FP8_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBPS
    # Counter-measured HBM bytes per launch, when every shape of the kernel
    # has a summary taken with the current kernel sources.
    measured = [read_traffic(preps[i].wl.name, args.scales) for i in idx]
    traffic = float(np.mean(measured)) if measured and all(x is not None for x in measured) else None
    # Counter-measured MFMA-busy fraction (matrix-core busy cycles over elapsed
    # cycles x SIMDs, at the clock the GPU actually ran), same condition.
    busy = [read_mfma_busy(preps[i].wl.name, args.scales) for i in idx]
    mfma_busy = float(np.mean(busy)) if busy and all(x is not None for x in busy) else None
    med_us = None
    if medians is not None:
        med_us = float(np.mean([medians[preps[i].wl.name] for i in idx]))
    roofline = {
        "bound": "mfma" if mfma_bound else "hbm",
        "achieved": round(achieved, 1),
        "peak": peak,
        "unit": "TFLOP/s" if mfma_bound else "GB/s",
        "frac": round(achieved / peak, 4),
        "traffic": round(traffic) if traffic is not None else None,
        "mfma_busy_frac": round(mfma_busy, 4) if mfma_busy is not None else None,
        "traffic_source": ([os.path.relpath(traffic_path(preps[i].wl.name, args.scales), os.path.dirname(PROFILES))
                            for i in idx]
                           if traffic is not None else None),
        "kernel": key,
        "launches_averaged": len(idx) * args.steps,
        "mean_algorithmic_bytes_per_launch": mean_bytes,
        "mean_algorithmic_flops_per_launch": mean_flops,
        "mean_launch_us": round(mean_dur * 1e6, 3),
        "rocprof_median_us": round(med_us, 3) if med_us is not None else None,
        "frac_from_rocprof_median": (round((mean_flops / (med_us * 1e-6) / 1e12 if mfma_bound
                                            else mean_bytes / (med_us * 1e-6) / 1e9) / peak, 4)
                                     if med_us is not None else None),
    }
    copies = [len(p.b) for p in preps]
    step_bytes = sum(p.bytes for p in preps)
    vs = None
    if all(pages_key(p.wl) is not None for p in preps):
        page_t = sum(p.flops / (PAGES_TFLOPS[pages_key(p.wl)] * 1e12) for p in preps)
        vs = round(value / (step_flops / page_t / 1e12), 4)
    del preps
    torch.cuda.empty_cache()

    # Per-shape records, one workload at a time (event-timed here; the
    # rocprofv3 median is the primary time where present).
    per_shape = []
    for w in shape_wls:
        if w.name in head_shape_ms:
            i = [h.name for h in headline].index(w.name)
            p = Prepared(dg, torch, w, args.scales)
            ev_ms, q_ms = head_shape_ms[w.name], head_quant_ms[i]
        else:
            p = Prepared(dg, torch, w, args.scales)
            _, g_ms = time_steps(dg, torch, [p], max(5, args.steps // 2), 2)
            ev_ms, q_ms = float(np.mean(g_ms[:, 0])), time_quant(dg, torch, p)
        med = medians.get(w.name) if medians else None
        per_shape.append(shape_record(p, ev_ms * 1e-3, q_ms, med))
        if args.workload in ("all", "pages"):
            print(json.dumps(per_shape[-1]), file=sys.stderr, flush=True)
        del p
        torch.cuda.empty_cache()

    head = headline[0]
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs,
        "vs_baseline_note": ("value / the pages' H800 GEMM-only TFLOPS for the same shapes (context on other "
                             "hardware, not the target; the step here also quantises the activations)"
                             if vs is not None else None),
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": "dense_decode_sweep_m128" if len(headline) > 1 else head.name,
            "layout": head.layout,
            "groups": head.groups,
            "m_per_group": head.m,
            "nk_pairs": [[w.n, w.k] for w in headline],
            "step": "dg_quant_1x128(A) + GEMM; weights quantised once before timing",
            "scales": args.scales,
            "weight_rotation_copies": copies,
            "num_cus": dg.dg_get_num_cus(),
        },
        "step_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": roofline,
        "per_shape_timing": {"primary": median_note if medians else None,
                             "secondary": "mean over event-bracketed launches in this process "
                                          "(includes ~1 us of dispatch per launch)"},
        "per_shape": per_shape,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(headline, args.cpu_seconds, args.scales)
    print(json.dumps(result), flush=True)
    return 0


def shape_record(p, t_events, quant_ms, median_us=None):
    """One shape's figures.  Time: the rocprofv3 median when given, else the
    event-timed mean (both are recorded)."""
    t = median_us * 1e-6 if median_us is not None else t_events
    tflops = p.flops / t / 1e12
    gbps = p.bytes / t / 1e9
    key = pages_key(p.wl)
    return {
        "pages_h800_tflops": PAGES_TFLOPS[key] if key else None,
        "vs_pages": round(tflops / PAGES_TFLOPS[key], 3) if key else None,
        "workload": p.wl.name,
        "layout": p.wl.layout,
        "groups": p.wl.groups,
        "m_valid": p.m_valid,
        "n": p.wl.n,
        "k": p.wl.k,
        "gemm_us": round(t * 1e6, 3),
        "gemm_us_source": "rocprofv3 median" if median_us is not None else "events mean",
        "gemm_us_rocprof_median": round(median_us, 3) if median_us is not None else None,
        "gemm_us_events_mean": round(t_events * 1e6, 3),
        "tflops": round(tflops, 2),
        "gbps": round(gbps, 1),
        "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
        "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "scale_bytes": p.sf_bytes,
        "quant_1x128_us": round(quant_ms * 1e3, 3),
        "traffic_bytes": _round_or_none(read_traffic(p.wl.name, p.scales)),
        "mfma_busy_frac": _round_or_none(read_mfma_busy(p.wl.name, p.scales), 4),
        "config": p.config,
    }


def _round_or_none(x, nd=0):
    """Counter-summary figure for the record: None when there is no summary
    taken with the current kernel sources."""
    if x is None:
        return None
    return round(x, nd) if nd else round(x)


if __name__ == "__main__":
    sys.exit(main())
