"""Host logic of bench.py, on the CPU: the algorithmic byte counts the
rooflines divide by, the normalisation of profiler counters (calibration by
the plain copies, per-dispatch medians, busy fractions), the timed-region
windowing of a kernel trace and the source-digest gate on recorded counters.
Synthetic profiler files stand in for rocprofv3 output; every expected value
is worked out by hand in the test."""
import csv
import os

import pytest

import bench

COPY_BYTES = bench.COPY_CAL_BYTES


def test_gemv_bytes_match_the_scope_table():
    # bits N K / 8 + scales 4 N K / 128 + x 4 K + y 4 N (the decode configs'
    # algorithmic bytes: ffn_gate and ffn_down 14,016,512, ssm_out 4,960,256,
    # tiny 46,080)
    assert bench.gemv_bytes(17408, 5120) == 14_016_512
    assert bench.gemv_bytes(5120, 17408) == 14_016_512
    assert bench.gemv_bytes(5120, 6144) == 4_960_256
    assert bench.gemv_bytes(256, 1024) == 46_080
    # f16 scales: two bytes per 128 weights instead of four
    assert bench.gemv_bytes(17408, 5120, scale_bytes=2) == 14_016_512 - 17408 * 40 * 2


@pytest.mark.parametrize("N,parts", [(17408, 16), (7, 16), (1, 1), (100, 3)])
def test_split_rows_partitions(N, parts):
    s = bench._split_rows(N, parts)
    assert s[0][0] == 0 and s[-1][1] == N
    assert all(a < b for a, b in s)
    assert all(s[i][1] == s[i + 1][0] for i in range(len(s) - 1))
    assert len(s) == min(N, parts)


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)
    with open(os.path.join(d, "run_agent_info.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Simd_Count", "Num_Xcc", "Cu_Count",
                                          "Max_Engine_Clk_Fcompute"])
        w.writeheader()
        w.writerow({"Name": "gfx950", "Simd_Count": 1024, "Num_Xcc": 8, "Cu_Count": 256,
                    "Max_Engine_Clk_Fcompute": 2400})


def _kv(path):
    kv = {}
    for line in open(path):
        if not line.startswith("#") and ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_gemm_counter_summary_normalisation(tmp_path):
    kern = "pq1::(anonymous namespace)::gemm_xg_kernel(unsigned short const*, ...)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE: the copies read 2 x 64 KiB of counter per 256 MiB copied
    # (factor 2048 bytes per KiB); the GEMM dispatches read 100, 120, 110 KiB
    fetch = [dict(Dispatch_Id=i, Kernel_Name=kern, Counter_Name="FETCH_SIZE", Counter_Value=v,
                  Start_Timestamp=0, End_Timestamp=1) for i, v in ((1, 100), (2, 120), (3, 110))]
    fetch += [dict(Dispatch_Id=10 + i, Kernel_Name=copy, Counter_Name="FETCH_SIZE",
                   Counter_Value=COPY_BYTES / 2048.0 / 2, Start_Timestamp=0, End_Timestamp=1)
              for i in range(3)]
    # split over two instances: must be summed per dispatch
    fetch += [dict(Dispatch_Id=10 + i, Kernel_Name=copy, Counter_Name="FETCH_SIZE",
                   Counter_Value=COPY_BYTES / 2048.0 / 2, Start_Timestamp=0, End_Timestamp=1)
              for i in range(3)]
    write = [dict(Dispatch_Id=i, Kernel_Name=kern, Counter_Name="WRITE_SIZE", Counter_Value=50,
                  Start_Timestamp=0, End_Timestamp=1) for i in (1, 2, 3)]
    write += [dict(Dispatch_Id=10 + i, Kernel_Name=copy, Counter_Name="WRITE_SIZE",
                   Counter_Value=COPY_BYTES / 1024.0, Start_Timestamp=0, End_Timestamp=1)
              for i in range(3)]
    # SQ pass: 2 dispatches of 1 ms; GRBM_GUI_ACTIVE 8 XCCs x 2e6 cycles (2 GHz);
    # MFMA busy 1024 SIMDs x 1e6 cycles (half the time), LDS active 256 CUs x 5e5
    sq = []
    for i in (1, 2):
        vals = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 1e6, "SQ_INSTS_MFMA": 1000.0,
                "SQ_INSTS_VALU": 6000.0, "SQ_INSTS_LDS": 1000.0, "SQ_LDS_IDX_ACTIVE": 256 * 5e5,
                "SQ_LDS_BANK_CONFLICT": 7.0, "SQ_WAIT_INST_LDS": 0.0, "GRBM_GUI_ACTIVE": 8 * 2e6}
        for c, v in vals.items():
            sq.append(dict(Dispatch_Id=i, Kernel_Name=kern, Counter_Name=c, Counter_Value=v,
                           Start_Timestamp=0, End_Timestamp=1_000_000))
    dirs = [str(tmp_path / n) for n in ("fetch", "write", "sq")]
    for d, rows in zip(dirs, (fetch, write, sq)):
        _write_counters(d, rows)
    out = str(tmp_path / "summary.txt")
    bench.summarize_gemm_pmc(*dirs, out)
    kv = _kv(out)
    assert float(kv["fetch_bytes_per_launch"]) == pytest.approx(110 * 2048.0)  # median 110 KiB
    assert float(kv["write_bytes_per_launch"]) == pytest.approx(50 * 1024.0)   # factor 1
    assert float(kv["mfma_busy_frac"]) == pytest.approx(0.5)
    assert float(kv["lds_active_frac"]) == pytest.approx(0.25)
    assert float(kv["valu_insts_per_mfma (MFMA included)"]) == pytest.approx(6.0)
    assert float(kv["lds_insts_per_mfma"]) == pytest.approx(1.0)
    assert float(kv["effective_clock_ghz"]) == pytest.approx(2.0)
    assert kv["source_sha256"] == bench.kernel_source_digest(bench.GEMM_KERNEL_SOURCES)


def test_trace_summary_keeps_only_marked_regions(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    k = "pq1::(anonymous namespace)::gemm_xg_kernel(int)"
    mark = "mark_kernel(void)"
    # a warm-up launch (outside), region 1: two launches of 2 and 4 us,
    # a launch between the regions (outside), region 2: one launch of 10 us
    rows = [(0, 50_000, k), (100_000, 100_500, mark), (101_000, 103_000, k),
            (104_000, 108_000, k), (109_000, 109_500, mark), (110_000, 170_000, k),
            (200_000, 200_500, mark), (201_000, 211_000, k), (212_000, 212_500, mark)]
    with open(d / "bench_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Start_Timestamp", "End_Timestamp", "Kernel_Name"])
        w.writerows(rows)
    log = tmp_path / "bench.err"
    log.write_text("[timed region] first\nnoise\n[timed region] second\n")
    out = tmp_path / "trace.md"
    bench.summarize_trace(str(d), str(out), "test", str(log))
    lines = [l for l in out.read_text().splitlines() if l.startswith("| first") or
             l.startswith("| second")]
    assert len(lines) == 2
    first = [c.strip() for c in lines[0].split("|")[1:-1]]
    second = [c.strip() for c in lines[1].split("|")[1:-1]]
    assert first[0] == "first" and first[2] == "2" and float(first[6]) == pytest.approx(3.0)
    assert second[0] == "second" and second[2] == "1" and float(second[4]) == pytest.approx(10.0)
    assert "inside the 2 marked timed regions" in out.read_text()


def test_recorded_gemm_counters_gated_by_source_digest(tmp_path, monkeypatch):
    good = bench.kernel_source_digest(bench.GEMM_KERNEL_SOURCES)
    p = tmp_path / "counters.txt"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "GEMM_COUNTER_FILE", "counters.txt")
    # the digest is computed from the sources under ROOT, which now points
    # at the temporary directory: keep the repository's value
    monkeypatch.setattr(bench, "kernel_source_digest", lambda sources=None: good)
    p.write_text(f"# header\nsource_sha256: {good}\nmfma_busy_frac: 0.55\n")
    kv = bench.recorded_gemm_counters()
    assert kv is not None and kv["mfma_busy_frac"] == "0.55"
    p.write_text("source_sha256: 0000\nmfma_busy_frac: 0.55\n")
    assert bench.recorded_gemm_counters() is None
    p.unlink()
    assert bench.recorded_gemm_counters() is None
