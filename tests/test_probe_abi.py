"""libdg_probe.so (the register-only loop probe the benchmark runs) loads,
exports what include/dg_probe.h declares, and rejects bad arguments on the
host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "moe_grouped_gemm_02_amd", "libdg_probe.so")
HEADER = os.path.join(ROOT, "include", "dg_probe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_exports_every_declared_function(lib):
    text = open(HEADER).read()
    names = re.findall(r"^int\s+(dg_\w+)\s*\(", text, flags=re.M)
    assert names == ["dg_probe_loop", "dg_probe_mfma_per_iter"]
    for n in names:
        assert hasattr(lib, n), n


def test_mfma_counts_and_argument_checks(lib):
    lib.dg_probe_loop.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    assert [lib.dg_probe_mfma_per_iter(m) for m in (0, 1, 2, 3, -1)] == [16, 32, 32, -1, -1]
    buf = ctypes.create_string_buffer(64)  # never dereferenced: every call below fails its checks
    p = ctypes.cast(buf, ctypes.c_void_p)
    bad = [(3, 8, 256, 10, p, p), (0, 6, 256, 10, p, p), (0, 8, 0, 10, p, p), (0, 8, 65536, 10, p, p),
           (0, 8, 256, 0, p, p), (0, 8, 256, 10, None, p), (0, 8, 256, 10, p, None)]
    for args in bad:
        assert lib.dg_probe_loop(*args, None) == -1, args
