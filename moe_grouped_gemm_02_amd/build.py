"""Ahead-of-time build of libdg.so for gfx950 (run on the host; no GPU needed).

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
LIB = os.path.join(HERE, "libdg.so")
SOURCES = ["dg_api.hip", "dg_quant.hip", "dg_gemm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs, where the promotion FMAs read them (no AGPR copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def build(verbose: bool = False, extra=None) -> str:
    """Compile libdg.so in-tree and return its path; raises on failure."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
