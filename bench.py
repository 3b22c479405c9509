#!/usr/bin/env python3
"""Benchmark of the fine-grained-scaled FP8 GEMM path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input: for
every shape of the workload, quantise the bf16 activations per 1x128 tile
(dg_quant_1x128) and run the GEMM (dg_fp8_gemm_nt, or the grouped entry
points) on weights that were quantised per 128x128 block once, before timing
(weights are converted offline, once per weight).

The default workload is the dense decode sweep M = 128 over the six (N, K)
pairs of DeepSeek-V3 shapes.  `--workload all` also measures every other
workload shape (one line per shape on stderr, and a per-shape table in the
JSON line).

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
    p.add_argument("--workload", default="decode128",
                   help="decode128 (default) | all | a workload name from synth.workloads()")
    p.add_argument("--scales", choices=("fp32", "ue8m0"), default="fp32",
                   help="scale format: fp32 (default) or power-of-two exponent bytes (UE8M0)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work for the oracle sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain device copy of known size (for counter calibration)")
    p.add_argument("--launches-only", metavar="WORKLOAD",
                   help="only quantise and launch this workload's GEMM --reps times, no timing "
                        "(the program rocprofv3 --pmc runs for the traffic counters)")
    p.add_argument("--reps", type=int, default=5)
    p.add_argument("--write-mfma", metavar="PMC_CSV",
                   help="with --launches-only W: write profiles/gemm_kernel_W_mfma.txt from a counter pass "
                        "over the MFMA counters (see write_mfma)")
    p.add_argument("--num-cus", type=int, default=256, help="CUs of the measured GPU, for --write-mfma")
    p.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                   help="write the traffic summary for --launches-only's workload from four rocprofv3 "
                        "counter_collection.csv files (no GPU needed)")
    return p.parse_args(argv)


# --------------------------------------------------------------- workloads --

def select_workloads(name):
    import synth
    wls = synth.workloads()
    extra = synth.pages_workloads() + synth.extra_workloads()
    if name == "decode128":
        return [w for w in wls if w.layout == "dense" and w.m == 128]
    if name == "all":
        return wls + extra
    if name == "pages":  # every row of the pages' performance tables
        return [w for w in wls + extra if pages_key(w) is not None]
    pick = [w for w in wls + extra if w.name == name]
    if not pick:
        raise SystemExit(f"unknown workload {name}; choose from decode128, all, pages, "
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

    Sample: for each shape, all M rows of A (at most 256) against the first
    1024 columns of B (eight 128-row weight blocks).  The activations are
    quantised inside the timed region, as in the GPU step; the weights are
    quantised before it, as in the GPU step.  The shapes are visited in turn,
    repeatedly, until about target_s seconds of oracle work are done.
    Rate = sample flops / oracle seconds.
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

    samples = []
    for wl in wls:
        m = wl.m if wl.layout == "dense" else min(wl.m, 256)
        ncols = min(wl.n, 1024)
        xa = synth.bf16_normal((m, wl.k), wl.seed_a)
        qb, sfb = quant_b(synth.bf16_normal((ncols, wl.k), wl.seed_b))
        samples.append((wl, m, ncols, xa, qb, sfb))
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
    names = ", ".join(f"{wl.name}[:{m}, :{nc}]" for wl, m, nc, *_ in samples)
    return {
        "value": flops / secs / 1e12,
        "unit": "TFLOPS",
        "cores": 1,
        "kind": "oracle",
        "sample": f"single-threaded numpy oracle (quantise A per 1x128 + fp64 blockwise GEMM), {runs} runs "
                  f"cycling over {names}; {secs:.1f} s of CPU work",
        "cpu_model": _cpu_model(),
        "host_cores": os.cpu_count(),
    }


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


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "moe_grouped_gemm_02_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_per_dispatch(path, counter, name_part):
    import csv
    sums = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                sums[r["Dispatch_Id"]] = sums.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not sums:
        raise SystemExit(f"no {counter} rows for kernels matching {name_part!r} in {path}")
    return float(np.median(list(sums.values()))), len(sums)


def traffic_path(workload, scales="fp32"):
    return os.path.join(PROFILES, f"gemm_kernel_{workload}{'_ue8m0' if scales == 'ue8m0' else ''}_traffic.txt")


def write_traffic(workload, scales, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    fetch, nf = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", "gemm_kernel")
    write, nw = _counter_per_dispatch(write_csv, "WRITE_SIZE", "gemm_kernel")
    cfetch, _ = _counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    cwrite, _ = _counter_per_dispatch(copy_write_csv, "WRITE_SIZE", "copyBuffer")
    fscale, wscale = COPY_BYTES / (cfetch * 1024), COPY_BYTES / (cwrite * 1024)
    traffic = fetch * 1024 * fscale + write * 1024 * wscale
    sflag = " --scales ue8m0" if scales == "ue8m0" else ""
    lines = [
        f"workload={workload}",
        f"scales={scales}",
        f"kernel_source_sha256_16={kernel_source_hash()}",
        f"fetch_kib_per_dispatch={fetch:.1f}  (median of {nf} dispatches)",
        f"write_kib_per_dispatch={write:.1f}  (median of {nw} dispatches)",
        f"copy_fetch_kib={cfetch:.1f}  copy_write_kib={cwrite:.1f}  (plain copy of {COPY_BYTES} bytes each way)",
        f"fetch_scale={fscale:.4f}  write_scale={wscale:.4f}",
        f"traffic_bytes_per_launch={traffic:.0f}",
        "",
        "commands (from the repository root, REPO = its absolute path):",
        "  cd /tmp && export TMPDIR=/tmp",
        "  rocprofv3 --pmc FETCH_SIZE -f csv -d $REPO/gpurun_out/pmc_copy_f -o p -- python3 $REPO/bench.py --calibrate-copy",
        "  rocprofv3 --pmc WRITE_SIZE -f csv -d $REPO/gpurun_out/pmc_copy_w -o p -- python3 $REPO/bench.py --calibrate-copy",
        f"  rocprofv3 --pmc FETCH_SIZE -f csv -d $REPO/gpurun_out/pmc_f -o p -- python3 $REPO/bench.py --launches-only {workload}{sflag}",
        f"  rocprofv3 --pmc WRITE_SIZE -f csv -d $REPO/gpurun_out/pmc_w -o p -- python3 $REPO/bench.py --launches-only {workload}{sflag}",
        f"  python3 bench.py --launches-only {workload}{sflag} --write-traffic gpurun_out/pmc_f/p_counter_collection.csv "
        "gpurun_out/pmc_w/p_counter_collection.csv gpurun_out/pmc_copy_f/p_counter_collection.csv "
        "gpurun_out/pmc_copy_w/p_counter_collection.csv",
    ]
    path = traffic_path(workload, scales)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_INSTS_MFMA "
                 "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")
MI355X_XCDS = 8


def mfma_path(workload, scales="fp32"):
    return os.path.join(PROFILES, f"gemm_kernel_{workload}{'_ue8m0' if scales == 'ue8m0' else ''}_mfma.txt")


def write_mfma(workload, scales, pmc_csv, num_cus):
    """MFMA-busy fraction of one workload's GEMM launches from a counter pass:
    SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (GRBM_GUI_ACTIVE per XCD x
    SIMDs), medians over the dispatches; plus the MFMA op count against the
    algorithmic flops."""
    busy, nd = _counter_per_dispatch(pmc_csv, "SQ_VALU_MFMA_BUSY_CYCLES", "gemm_kernel")
    gui, _ = _counter_per_dispatch(pmc_csv, "GRBM_GUI_ACTIVE", "gemm_kernel")
    mops, _ = _counter_per_dispatch(pmc_csv, "SQ_INSTS_VALU_MFMA_MOPS_F8", "gemm_kernel")
    simds = 4 * num_cus
    frac = busy / (gui / MI355X_XCDS * simds)
    sflag = " --scales ue8m0" if scales == "ue8m0" else ""
    lines = [
        f"workload={workload}",
        f"scales={scales}",
        f"kernel_source_sha256_16={kernel_source_hash()}",
        f"mfma_busy_cycles={busy:.6g}  (SQ_VALU_MFMA_BUSY_CYCLES, median of {nd} dispatches, all SIMDs)",
        f"grbm_gui_active={gui:.6g}  (summed over {MI355X_XCDS} XCDs)",
        f"simds={simds}",
        f"mfma_busy_frac={frac:.4f}",
        f"mfma_flops={mops * 512:.6g}  (SQ_INSTS_VALU_MFMA_MOPS_F8 x 512)",
        "",
        "commands (from the repository root, REPO = its absolute path):",
        "  cd /tmp && export TMPDIR=/tmp",
        f"  rocprofv3 --pmc {MFMA_COUNTERS} -f csv -d $REPO/gpurun_out/pmcm -o p -- python3 $REPO/bench.py --launches-only {workload}{sflag}",
        f"  python3 bench.py --launches-only {workload}{sflag} --write-mfma gpurun_out/pmcm/p_counter_collection.csv",
    ]
    path = mfma_path(workload, scales)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


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
            raise SystemExit("--write-traffic needs --launches-only WORKLOAD")
        write_traffic(args.launches_only, args.scales, *args.write_traffic)
        return 0
    if args.write_mfma:
        if not args.launches_only:
            raise SystemExit("--write-mfma needs --launches-only WORKLOAD")
        write_mfma(args.launches_only, args.scales, args.write_mfma, args.num_cus)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
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
        wl = {w.name: w for w in synth.workloads() + synth.pages_workloads() + synth.extra_workloads()}[args.launches_only]
        p = Prepared(dg, torch, wl, args.scales)
        for r in range(args.reps):
            p.quant(dg)
            p.gemm(dg, r)
        torch.cuda.synchronize()
        print(json.dumps({"launches": args.reps, "workload": wl.name, "config": p.config}))
        return 0

    wls = select_workloads(args.workload)
    headline = [w for w in wls if w.layout == "dense" and w.m == 128] or wls
    preps = [Prepared(dg, torch, w, args.scales) for w in headline]
    torch.cuda.synchronize()

    # Per-shape pass (not the benchmark value): every GEMM launch bracketed by
    # events, which also picks the dominant kernel - the GEMM configuration
    # with the most total time.
    _, shape_ms = time_steps(dg, torch, preps, args.steps, args.warmup)
    by_kernel = {}
    for i, p in enumerate(preps):
        by_kernel.setdefault(p.kernel_key, []).append(i)
    key = max(by_kernel, key=lambda k_: sum(float(np.sum(shape_ms[:, i])) for i in by_kernel[k_]))
    idx = by_kernel[key]

    # The timed pass: W warmup steps, then exactly K steps between two torch
    # events; only the dominant kernel's launches carry HIP events (each
    # event record costs the stream ~0.8 us, ~19 us per step if every launch
    # were bracketed).
    total_ms, gemm_ms = time_steps(dg, torch, preps, args.steps, args.warmup, instrument=idx)
    ms_per_step = total_ms / args.steps
    step_flops = sum(p.flops for p in preps)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    per_shape = []
    for i, p in enumerate(preps):
        t = float(np.mean(shape_ms[:, i])) * 1e-3
        per_shape.append(shape_record(p, t, time_quant(dg, torch, p)))

    extra = []
    if args.workload in ("all", "pages"):
        for w in wls:
            if w in headline:
                continue
            p = Prepared(dg, torch, w, args.scales)
            _, g_ms = time_steps(dg, torch, [p], max(5, args.steps // 2), 2)
            extra.append(shape_record(p, float(np.mean(g_ms[:, 0])) * 1e-3, time_quant(dg, torch, p)))
            print(json.dumps(extra[-1]), file=sys.stderr, flush=True)
            del p
            torch.cuda.empty_cache()

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
    }

    vs = None
    if headline and all(pages_key(w) is not None for w in headline):
        page_t = sum(p.flops / (PAGES_TFLOPS[pages_key(p.wl)] * 1e12) for p in preps)
        vs = round(value / (step_flops / page_t / 1e12), 4)

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
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": "dense_decode_sweep_m128" if len(headline) > 1 else headline[0].name,
            "m": headline[0].m,
            "nk_pairs": [[w.n, w.k] for w in headline],
            "step": "dg_quant_1x128(A) + GEMM per shape; weights quantised once before timing",
            "scales": args.scales,
            "weight_rotation_copies": [len(p.b) for p in preps],
            "num_cus": dg.dg_get_num_cus(),
        },
        "step_gbps": round(sum(p.bytes for p in preps) / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": roofline,
        "per_shape": per_shape + extra,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(headline, args.cpu_seconds, args.scales)
    print(json.dumps(result), flush=True)
    return 0


def shape_record(p, t, quant_ms):
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
        "tflops": round(tflops, 2),
        "gbps": round(gbps, 1),
        "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
        "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "scale_bytes": p.sf_bytes,
        "quant_1x128_us": round(quant_ms * 1e3, 3),
        "config": p.config,
    }


if __name__ == "__main__":
    sys.exit(main())
