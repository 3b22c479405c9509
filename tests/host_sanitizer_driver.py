"""Child process of test_host_sanitizers.py (not a test module itself).

Loads libdg_host_asan.so (the library with its host code built under
AddressSanitizer and UndefinedBehaviorSanitizer) with ctypes, takes every
entry point's signature from include/dg.h, and drives the host code that runs
without a GPU: argument checks and their error messages, tile planning and
workspace sizing for many shapes and CU counts, configuration strings into
small buffers, and the launch preparation up to the kernel launch, which
fails with DG_ERR_HIP on a machine without a GPU.  Device pointers are fake,
aligned addresses that the host code never dereferences.  A sanitizer report
aborts the process; otherwise the last line reads "host-sanitizer driver ok
calls=N".  Run with no torch import: only ctypes touches the library.

usage: python host_sanitizer_driver.py LIB HEADER
"""

import ctypes
import os
import re
import sys

FAKE = 1 << 24            # 16-byte aligned, never dereferenced on the host
BIG_WS = 1 << 40          # a workspace size larger than any need
STATUSES = {0, -1, -2, -3, -4, -5}
C_TYPES = {"int": ctypes.c_int, "int64_t": ctypes.c_int64, "size_t": ctypes.c_size_t}
CALLS = 0


def declarations(header):
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    out = {}
    for ret, name, args in re.findall(r"(int|size_t|int64_t|const char\*)\s+(dg_\w+)\s*\(([^)]*)\)\s*;", text):
        params = []
        for arg in " ".join(args.split()).split(","):
            arg = arg.strip()
            if arg in ("void", ""):
                continue
            ctype, pname = arg.rsplit(" ", 1)
            if pname.startswith("*"):
                ctype, pname = ctype + "*", pname[1:]
            params.append((ctype, pname))
        out[name] = (ret, params)
    return out


def bind(lib, decls):
    for name, (ret, params) in decls.items():
        fn = getattr(lib, name)
        fn.restype = ctypes.c_char_p if ret == "const char*" else C_TYPES[ret]
        fn.argtypes = [ctypes.c_void_p if "*" in t else C_TYPES[t] for t, _ in params]
    return lib


def up(x, a):
    return (x + a - 1) // a * a


def valid_args(name, params, s):
    """Arguments that pass every host check of entry point `name` for shape s."""
    m, n, k, g = s["m"], s["n"], s["k"], s["g"]
    a_mn = name.startswith(("dg_fp8_gemm_tn", "dg_fp8_gemm_tt"))
    b_mn = name.startswith(("dg_fp8_gemm_nn", "dg_fp8_gemm_tn"))
    rows = m
    vals = {
        "m": m, "n": n, "k": k, "m_total": m, "m_max": m, "num_groups": g, "expected_m": s.get("expected_m", 0),
        "lda": m if a_mn else k, "ldb": n if b_mn else k, "ldd": up(n, 8),
        "ld_sfa": up(rows, 4), "ld_sfb": up(n, 4), "ld_dsf": up(rows, 4),
        "workspace": FAKE, "workspace_bytes": BIG_WS, "stream": None,
        "rows": s.get("rows", m), "cols": s.get("cols", k),
    }
    if name.startswith("dg_quant"):
        vals["num_groups"] = 1
        vals["ld_sf"] = up(vals["cols"] if "_mn" in name else vals["rows"], 4)
    out = []
    for ctype, pname in params:
        if "*" in ctype:
            out.append(None if pname == "stream" else FAKE)
        else:
            out.append(vals[pname])
    return out


def call(fn, args):
    global CALLS
    CALLS += 1
    return fn(*args)


def check_status(lib, st, what):
    assert st in STATUSES, f"{what}: status {st}"
    msg = lib.dg_get_last_error_string()
    assert msg is not None
    if st != 0:
        assert msg, f"{what}: status {st} without a message"


GEMM_SHAPES = {
    "dense": [dict(m=128, n=7168, k=16384, g=1), dict(m=64, n=2048, k=7168, g=1), dict(m=4096, n=4096, k=7168, g=1),
              dict(m=16, n=128, k=128, g=1), dict(m=208, n=384, k=1024, g=1), dict(m=128, n=2112, k=7168, g=1)],
    "contiguous": [dict(m=1024, n=4096, k=7168, g=4), dict(m=128, n=256, k=128, g=1)],
    "masked": [dict(m=256, n=4096, k=7168, g=8, expected_m=e) for e in (0, 1, 64, 200)],
    "kgrouped": [dict(m=256, n=512, k=4096, g=4), dict(m=128, n=128, k=128, g=1)],
    "quant": [dict(m=0, n=0, k=0, g=1, rows=r, cols=c) for r, c in ((1, 128), (129, 7168), (4096, 1024), (128, 64))],
}


def family(name):
    if name.startswith("dg_quant"):
        return "quant"
    if name.startswith("dg_grouped_contiguous"):
        return "contiguous"
    if name.startswith("dg_grouped_masked"):
        return "masked"
    if name.startswith("dg_k_grouped"):
        return "kgrouped"
    return "dense"


def drive_entry(lib, name, params):
    fn = getattr(lib, name)
    fam = family(name)
    for s in GEMM_SHAPES[fam]:
        if "qout" in name and s["n"] % 128:
            continue
        if fam == "quant" and "_mn" in name and (s["rows"] % 128 or s["cols"] % 8):
            continue
        if fam == "quant" and "_mn" not in name and s["cols"] % 128:
            continue
        base = valid_args(name, params, s)
        st = call(fn, base)
        assert st == -5, f"{name} {s}: expected the launch to fail without a GPU, got {st}: " \
                         f"{lib.dg_get_last_error_string()}"
        # One argument at a time: null / misaligned pointers, odd sizes.
        for i, (ctype, pname) in enumerate(params):
            if "*" in ctype:
                tries = [0, FAKE + 1, FAKE + 4] if pname != "stream" else []
            elif ctype == "int":
                tries = [-1, 0, 1, 7, 127, 129, 1 << 20, 2**31 - 1, -2**31]
            elif ctype == "int64_t":
                tries = [-1, 0, 1, 4, 1 << 20, 1 << 40, 1 << 62, 2**63 - 16, 2**63 - 1, -2**63]
            else:
                tries = [0, 1]
            for v in tries:
                args = list(base)
                args[i] = v
                check_status(lib, call(fn, args), f"{name} {pname}={v}")


def drive_extremes(lib, decls, names):
    """Shapes at the edges of int: rejected (or empty) without overflow."""
    big = 2**31 - 1
    shapes = [dict(m=big, n=big, k=0, g=1), dict(m=big, n=128, k=0, g=big), dict(m=128, n=big, k=0, g=1),
              dict(m=big - big % 128, n=4096, k=0, g=1), dict(m=2**24, n=2**24, k=128, g=1),
              dict(m=1 << 20, n=7168, k=7168, g=64), dict(m=0, n=0, k=2**31 - 128, g=1),
              dict(m=0, n=0, k=0, g=1, rows=big, cols=big - big % 128), dict(m=0, n=0, k=0, g=1, rows=big - big % 128, cols=128),
              dict(m=0, n=0, k=0, g=1, rows=128, cols=big - big % 8), dict(m=0, n=0, k=0, g=1, rows=65535 * 128, cols=128)]
    for name in names:
        fn = getattr(lib, name)
        params = decls[name][1]
        for s in shapes:
            check_status(lib, call(fn, valid_args(name, params, s)), f"{name} {s}")


def drive_planning(lib):
    buf_sizes = [1, 2, 17, 64, 512]
    dims = [0, 1, 15, 64, 128, 129, 1000, 4096, 65536, 1 << 20, 2**31 - 1]
    ks = [0, 128, 7168, 16384, 1 << 20, 2**31 - 128]
    for layout in (0, 1, 2, 3, 8, 9, 10, 11, 4, -1, 12):
        for m in dims[::2]:
            for n in dims[1::2]:
                for k in ks[::2]:
                    for groups, em in ((1, 0), (4, 64), (64, 2**31 - 1)):
                        for cus in (1, 80, 256, 4096):
                            size = buf_sizes[(m + n + k + cus) % len(buf_sizes)]
                            buf = ctypes.create_string_buffer(size)
                            st = call(lib.dg_describe_config, [layout, m, n, k, groups, em, cus, buf, size])
                            check_status(lib, st, f"describe {layout} {m} {n} {k}")
                            if st == 0:
                                assert len(buf.value) < size
    for cus in (0, 1, 80, 256, 4096):
        assert lib.dg_set_num_cus(cus) == 0
        for m in dims:
            for n in dims[::3]:
                for k in ks:
                    for groups in (0, 1, 7, 4096, 2**31 - 1):
                        call(lib.dg_get_workspace_size, [m, n, k, groups])
    for v in (-1, 4097):
        check_status(lib, call(lib.dg_set_num_cus, [v]), f"set_num_cus {v}")
    # Forced configurations, well-formed or not ("variant:division:k_rotate").
    buf = ctypes.create_string_buffer(256)
    for forced in ("0", "6:4:1", "4:2", "99", "-1", "0:9999", "4:abc:7", ":", "::", "5:1:", "10:0:0", "3:-5"):
        os.environ["DG_FORCE_CONFIG"] = forced
        for layout, m, n, k, g in ((0, 128, 7168, 16384, 1), (2, 256, 4096, 7168, 8), (1, 1024, 4096, 7168, 4),
                                   (8, 64, 2048, 7168, 1), (3, 256, 512, 4096, 4), (0, 1, 1, 128, 1)):
            check_status(lib, call(lib.dg_describe_config, [layout, m, n, k, g, 0, 256, buf, 256]), f"forced {forced}")
            call(lib.dg_get_workspace_size, [m, n, k, g])
    os.environ.pop("DG_FORCE_CONFIG")
    for v in (-2**31, -1, 0, 1, 5, 2**31 - 1):
        call(lib.dg_get_sf_leading_dim, [v])
        call(lib.dg_get_ue8m0_sfb_leading_dim, [v])


def main():
    lib_path, header = sys.argv[1], sys.argv[2]
    decls = declarations(header)
    lib = bind(ctypes.CDLL(lib_path), decls)
    exported = [n for n in decls if not n.startswith("dg_get_") and n not in ("dg_set_num_cus", "dg_describe_config")]
    # The CU count normally comes from the device; without one, fix it.
    for env_cus in ("", "abc", "-3", "99999", "80"):
        os.environ["DG_NUM_CUS"] = env_cus
        call(lib.dg_get_num_cus, [])
    os.environ.pop("DG_NUM_CUS")
    assert lib.dg_set_num_cus(256) == 0
    os.environ["DG_DEBUG"] = "1"       # also format the planning line on stderr
    for name in exported:
        drive_entry(lib, name, decls[name][1])
    os.environ["DG_DEBUG"] = "0"
    drive_extremes(lib, decls, exported)
    drive_planning(lib)
    # The sanitizer runtime is live in this process: a freed heap block reads
    # as poisoned (without touching it).
    libc = ctypes.CDLL(None)
    libc.malloc.restype = ctypes.c_void_p
    libc.malloc.argtypes = [ctypes.c_size_t]
    libc.free.argtypes = [ctypes.c_void_p]
    poisoned = libc.__asan_address_is_poisoned
    poisoned.argtypes = [ctypes.c_void_p]
    block = libc.malloc(64)
    assert poisoned(block) == 0 and poisoned(block + 64) == 1
    libc.free(block)
    assert poisoned(block) == 1
    print(f"host-sanitizer driver ok calls={CALLS} entries={len(exported)}", flush=True)


if __name__ == "__main__":
    main()
