"""Ahead-of-time build of libdg.so for gfx950 (run on the host; no GPU needed).

build() also compiles libdg_host_asan.so, the same sources with the HOST code
instrumented by AddressSanitizer and UndefinedBehaviorSanitizer (device code
is compiled exactly as in libdg.so).  Nothing on the GPU path loads it: the
CPU tests drive its argument checks, tile planning and launch preparation in
a child process that preloads the sanitizer runtime.  Every source of both
libraries compiles in its own process at once (objects under _build/), then
each library is linked, so the second library adds little wall time.

build() also compiles libdg_probe.so from dg_probe.hip: a register-only
throughput probe of the GEMM inner loop's instruction mixes that the
benchmark runs (bench.py --probe-ceiling).  libdg.so does not contain it.

Every kernel is compiled for gfx950 only.  Flags:
* -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 VALU ops
  (v_pk_fma_f32 and friends) in the generated code;
* correctly rounded fp32 division and kept denormals: the quantiser's
  amax/448 and x/s are IEEE divisions, subnormal scales included.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdg.so")
ASAN_LIB = os.path.join(HERE, "libdg_host_asan.so")
# The register-only loop probe (include/dg_probe.h), a measurement tool the
# benchmark loads; the GEMM library does not contain it.
PROBE_LIB = os.path.join(HERE, "libdg_probe.so")
PROBE_SOURCES = ["dg_probe.hip"]
SOURCES = ["dg_api.hip", "dg_quant.hip", "dg_gemm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs, where the promotion FMAs read them (no AGPR copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]

# Host-side sanitizers only: every -fsanitize= goes to the host pass.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]

_NOISE = "packed-fp32-ops' is not a recognized feature"


def _run_all(cmds, verbose):
    """Run the commands at once; return (failures, notes) as text."""
    procs = []
    for label, cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((label, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed, notes = [], []
    for label, proc in procs:
        text, _ = proc.communicate()
        out = "\n".join(line for line in text.splitlines() if _NOISE not in line)
        if proc.returncode != 0:
            failed.append(f"hipcc failed for {label} ({proc.returncode}):\n{out}")
        elif out.strip():
            notes.append(out)
    return failed, notes


def build(verbose: bool = False, extra=None, host_asan: bool = True) -> str:
    """Compile libdg.so (and, unless host_asan is False, libdg_host_asan.so)
    in-tree and return the path of libdg.so; raises on failure."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    libs = [(LIB, "plain", list(extra or []), SOURCES), (PROBE_LIB, "plain", list(extra or []), PROBE_SOURCES)]
    if host_asan:
        libs.append((ASAN_LIB, "host_asan", [*(extra or []), *HOST_SANITIZE], SOURCES))
    compiles, links = [], []
    for lib, tag, flags, sources in libs:
        objs = []
        for src in sources:
            obj = os.path.join(OBJ_DIR, f"{os.path.splitext(src)[0]}.{tag}.o")
            objs.append(obj)
            compiles.append((f"{src} ({tag})", [HIPCC, *FLAGS, *flags, "-I", INCLUDE, "-I", CSRC, "-c",
                                                os.path.join(CSRC, src), "-o", obj]))
        links.append((os.path.basename(lib), [HIPCC, *FLAGS, *flags, "-shared", *objs, "-o", lib + ".tmp"]))
    failed, notes = _run_all(compiles, verbose)
    if not failed:
        failed, more = _run_all(links, verbose)
        notes += more
    if failed:
        raise RuntimeError("\n".join(failed))
    if verbose and notes:
        print("\n".join(notes))
    for lib, _, _, _ in libs:
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, host_asan="--no-host-asan" not in sys.argv))
