"""Pins for the benchmark's throughput accounting and the tile arithmetic,
against the numbers the pages print (CPU only).

* The pages' GB/s column equals (G*M*K + G*N*K + 2*G*M*N) bytes -- fp8 A,
  fp8 B and bf16 D -- divided by t = 2*G*M*N*K / TFLOPS, for every row of the
  three performance tables (DeepGEMM project introduction, section
  Performance; fixture tests/golden/deepgemm_perf_tables.csv).
* Unaligned block sizes (same page, section Optimisations, "unaligned block
  sizes"): M=256, N=7168 with 128x128 blocks gives 112 tiles; with BLOCK_N=112
  it gives 128.
"""

import csv
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "deepgemm_perf_tables.csv")


def _rows():
    with open(GOLDEN) as f:
        return list(csv.DictReader(line for line in f if not line.startswith("#")))


def test_fixture_has_the_three_tables():
    rows = _rows()
    assert len(rows) == 28
    assert {r["layout"] for r in rows} == {"dense", "contiguous", "masked"}


@pytest.mark.parametrize("row", _rows(), ids=lambda r: f"{r['layout']}-{r['groups']}x{r['m_per_group']}x{r['n']}x{r['k']}")
def test_bytes_formula_reproduces_pages_gbps(row):
    g, m, n, k = (int(row[x]) for x in ("groups", "m_per_group", "n", "k"))
    tflops, gbps = float(row["tflops"]), float(row["gbps"])
    flops = bench.algorithmic_flops(g * m, n, k)
    t = flops / (tflops * 1e12)
    derived = bench.algorithmic_bytes(g * m, n, k, g) / t / 1e9
    assert abs(derived - gbps) / gbps < 0.005


def test_headline_decode_context_number():
    # Aggregate H800 TFLOPS over the six M=128 dense shapes (time-weighted),
    # the context number bench.py divides by for vs_baseline.
    rows = [r for r in _rows() if r["layout"] == "dense" and r["m_per_group"] == "128"]
    flops = sum(bench.algorithmic_flops(128, int(r["n"]), int(r["k"])) for r in rows)
    secs = sum(bench.algorithmic_flops(128, int(r["n"]), int(r["k"])) / (float(r["tflops"]) * 1e12) for r in rows)
    assert 530 < flops / secs / 1e12 < 555
    for r in rows:
        assert bench.PAGES_TFLOPS[("dense", 1, 128, int(r["n"]), int(r["k"]))] == int(r["tflops"])


def test_unaligned_block_example():
    def tiles(m, n, bm, bn):
        return -(-m // bm) * -(-n // bn)
    assert tiles(256, 7168, 128, 128) == 112
    assert tiles(256, 7168, 128, 112) == 128


def test_library_tile_count_matches_the_example():
    dg = pytest.importorskip("moe_grouped_gemm_02_amd", reason="libdg.so not built")
    os.environ["DG_FORCE_CONFIG"] = "1:1"  # the 128x128 tile, no split
    try:
        desc = dg.dg_describe_config(dg.LAYOUT_DENSE, 256, 7168, 7168, 1, 132)
    finally:
        del os.environ["DG_FORCE_CONFIG"]
    assert "bm=128 bn=128" in desc and "tiles=112" in desc


def test_counter_summaries_split_dispatches_per_workload(tmp_path, monkeypatch):
    # One rocprofv3 --pmc pass over bench.py --launches-only W1,W2 --reps 3
    # sees 6 GEMM dispatches in order; each workload's summary takes the
    # median of its own 3, scaled by the copy calibration.
    import csv
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))

    def write_csv(path, counter, kernel, values):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for d, v in enumerate(values, start=10):
                for part in (0.25, 0.75):  # two counter instances per dispatch, summed
                    w.writerow({"Dispatch_Id": d, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": v * part})
                w.writerow({"Dispatch_Id": d + 100, "Kernel_Name": "quant_1x128_kernel", "Counter_Name": counter,
                            "Counter_Value": 1e9})

    f, wr, cf, cw = (str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    write_csv(f, "FETCH_SIZE", "gemm_kernel<x>", [100, 300, 200, 1000, 1200, 1100])
    write_csv(wr, "WRITE_SIZE", "gemm_kernel<x>", [10, 10, 10, 50, 50, 50])
    write_csv(cf, "FETCH_SIZE", "__amd_rocclr_copyBuffer", [bench.COPY_BYTES / 1024 / 2])
    write_csv(cw, "WRITE_SIZE", "__amd_rocclr_copyBuffer", [bench.COPY_BYTES / 1024])
    bench.write_traffic(["w1", "w2"], "fp32", 3, f, wr, cf, cw)
    got = {}
    for wl in ("w1", "w2"):
        fields = dict(line.split("=", 1) for line in open(bench.traffic_path(wl)) if "=" in line and not line.startswith(" "))
        got[wl] = float(fields["traffic_bytes_per_launch"].split()[0])
    assert got == {"w1": (200 * 2 + 10) * 1024, "w2": (1100 * 2 + 50) * 1024}
    with pytest.raises(SystemExit):
        bench.write_traffic(["w1", "w2", "w3"], "fp32", 3, f, wr, cf, cw)


def test_stall_summary_shares(tmp_path, monkeypatch):
    # Two --pmc passes over two workloads x 1 launch: the summary divides the
    # wave-state counters by SQ_WAVE_CYCLES and the busy counters by the
    # kernel's cycles per XCD times the units.
    import csv
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    values_a = {"SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 300.0, "SQ_WAIT_INST_ANY": 400.0, "SQ_WAIT_INST_LDS": 40.0,
                "SQ_ACTIVE_INST_VALU": 190.0, "SQ_ACTIVE_INST_LDS": 30.0, "SQ_INSTS_VALU": 600.0,
                "SQ_INSTS_LDS": 100.0, "GRBM_GUI_ACTIVE": 8 * 2000.0, "TA_TA_BUSY": 256 * 500.0}
    values_b = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 1000.0, "SQ_INSTS_MFMA": 100.0, "SQ_INSTS_SALU": 250.0,
                "SQ_ACTIVE_INST_SCA": 50.0, "SQ_LDS_CMD_FIFO_FULL": 256 * 100.0, "SQ_LDS_DATA_FIFO_FULL": 0.0,
                "SQ_WAVES": 2048.0, "GRBM_GUI_ACTIVE": 8 * 2000.0}
    assert set(values_a) == set(bench.STALL_COUNTERS[0].split())
    assert set(values_b) == set(bench.STALL_COUNTERS[1].split())

    def write_csv(path, values):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for d, scale in ((1, 1.0), (2, 2.0)):  # the second workload doubles every count
                for c, v in values.items():
                    w.writerow({"Dispatch_Id": d, "Kernel_Name": "gemm_kernel<x>", "Counter_Name": c,
                                "Counter_Value": v * scale})

    a, b = str(tmp_path / "a.csv"), str(tmp_path / "b.csv")
    write_csv(a, values_a)
    write_csv(b, values_b)
    bench.write_stalls(["w1", "w2"], "fp32", 1, a, b, 256)
    for wl in ("w1", "w2"):
        text = open(bench.stalls_path(wl)).read()
        fields = {}
        for line in text.splitlines():
            for tok in line.split():
                if "=" in tok:
                    k, v = tok.split("=", 1)
                    fields[k] = v
        assert float(fields["wait_any"]) == pytest.approx(0.3)
        assert float(fields["wait_inst_any"]) == pytest.approx(0.4)
        assert float(fields["active_valu"]) == pytest.approx(0.19)
        assert float(fields["active_sca"]) == pytest.approx(0.05)
        assert float(fields["mfma_busy_frac"]) == pytest.approx(0.5)
        assert float(fields["ta_busy_frac"]) == pytest.approx(0.25)
        assert float(fields["lds_cmd_fifo_full_frac"]) == pytest.approx(0.05)
        assert float(fields["valu_insts_per_mfma"]) == pytest.approx(5.0)
        assert float(fields["salu_insts_per_mfma"]) == pytest.approx(2.5)


def test_kernel_source_hash_ignores_comments_only():
    # Counter summaries carry the hash of the kernel code they were taken
    # from; editing a comment keeps it, editing code changes it.
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    assert bench._strip_comments(code) == bench._strip_comments(code.replace("one more", "add one"))
    assert bench._strip_comments(code) == bench._strip_comments(code.replace("block\n comment", "other"))
    assert bench._strip_comments(code) != bench._strip_comments(code.replace("x + 1", "x + 2"))
    assert "one more" not in bench._strip_comments(code) and "return x + 1;" in bench._strip_comments(code)
