"""Per-kernel resource report of the gfx950 build (registers, LDS, scratch,
occupancy), taken from the compiler's kernel-resource-usage remarks.

Compiles each kernel source for the device only, with the flags of build.py,
and prints a markdown table: one row per kernel instance.  A kernel that
spills or uses scratch shows it here first, before any timing does.

usage: python3 moe_grouped_gemm_02_amd/resource_usage.py [source.hip ...]
"""

import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

from moe_grouped_gemm_02_amd import build as B  # noqa: E402

CXXFILT = "c++filt"
KERNEL_SOURCES = ["dg_gemm.hip", "dg_quant.hip"]
FIELDS = [("VGPRs", "VGPRs"), ("AGPRs", "AGPRs"), ("TotalSGPRs", "SGPRs"),
          ("ScratchSize [bytes/lane]", "scratch B/lane"), ("VGPRs Spill", "VGPR spill"),
          ("SGPRs Spill", "SGPR spill"), ("LDS Size [bytes/block]", "static LDS B"),
          ("Occupancy [waves/SIMD]", "waves/SIMD")]


def remarks(src):
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [B.HIPCC, *B.FLAGS, "-I", B.INCLUDE, "-I", B.CSRC, "--cuda-device-only", "-c",
               os.path.join(B.CSRC, src), "-o", os.path.join(tmp, "k.o"),
               "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp)
    if res.returncode != 0:
        raise RuntimeError(res.stderr[-4000:])
    return parse(res.stderr)


def parse(text):
    """{mangled kernel name: {remark field: value}} from the remark lines."""
    kernels, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([^:]+): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels


def demangle(names):
    if not names:
        return {}
    out = subprocess.run([CXXFILT], input="\n".join(names), capture_output=True, text=True, check=True).stdout
    return dict(zip(names, out.splitlines()))


def short(name):
    name = name.replace("(anonymous namespace)::", "").replace("dg::", "")
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\([^()]*\)$", "", name)  # drop the parameter list


def main(sources):
    print("| source | kernel instance | " + " | ".join(h for _, h in FIELDS) + " |")
    print("|---|---|" + "---:|" * len(FIELDS))
    for src in sources:
        ks = remarks(src)
        names = demangle(sorted(ks))
        for mangled in sorted(ks, key=lambda x: names[x]):
            v = ks[mangled]
            print(f"| {src} | `{short(names[mangled])}` | " + " | ".join(str(v.get(f, "")) for f, _ in FIELDS) + " |")


if __name__ == "__main__":
    main(sys.argv[1:] or KERNEL_SOURCES)
